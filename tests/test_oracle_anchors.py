"""Pins the oracle's coded anchors (tables version 2, blobs version 3): the
8-bit anchors of every group range-coded with one 256-symbol table per (kv,
layer), counted over the tensor the tables are built from (CacheGen blog,
section 2.1 pseudocode: the quantised anchor, then arithmetic coding).

The range coder on a 256-symbol alphabet is pinned by brute force over every
string of up to two symbols, round trips under any trailing bytes and the
information-theoretic bounds; the anchor tables by a numpy recount of the
anchors; the container by decoding each anchor stream back to the raw anchors
and by the whole blob decoding to exactly what the raw-anchor blob decodes to."""
import itertools

import numpy as np
import pytest

import synth

PTOT = 1 << 15


def cost_bits(sym, freq):
    f = np.asarray(freq, np.float64)
    return float(-np.log2(f[np.asarray(sym)] / PTOT).sum())


def tables_256(rng):
    uniform = np.full(256, 128, np.uint16)
    geo = np.maximum(1, (PTOT * 0.5 ** (np.arange(256) / 12.0))).astype(np.float64)
    geo = np.floor(geo / geo.sum() * (PTOT - 256)).astype(np.int64) + 1
    geo[0] += PTOT - geo.sum()
    extreme = np.ones(256, np.int64)
    extreme[137] = PTOT - 255
    rnd = rng.integers(1, 400, 256).astype(np.int64)
    rnd = np.floor(rnd / rnd.sum() * (PTOT - 256)).astype(np.int64) + 1
    rnd[rng.integers(256)] += PTOT - rnd.sum()
    return {"uniform": uniform, "geometric": geo.astype(np.uint16),
            "extreme": extreme.astype(np.uint16), "random": rnd.astype(np.uint16)}


def test_tables_are_valid(oracle_lib):
    for name, f in tables_256(np.random.default_rng(0)).items():
        assert f.size == 256 and int(f.astype(np.int64).sum()) == PTOT and f.min() >= 1, name


def test_every_string_of_up_to_two_symbols_round_trips(oracle_lib):
    f = tables_256(np.random.default_rng(1))["geometric"]
    seen = {}
    for n in (1, 2):
        for s in itertools.product(range(256), repeat=n):
            data = oracle_lib.rc_encode(np.array(s, np.uint8), f)
            for trail in (b"", b"\x00" * 4, b"\xff" * 4):
                back, _, bad = oracle_lib.rc_decode(data + trail, n, f)
                assert not bad and tuple(back) == s
            assert (n, data) not in seen  # injective for a fixed length
            seen[(n, data)] = s
            bits = 8 * len(data)
            c = cost_bits(s, f)
            assert c <= bits <= c + 16 + 1e-9


@pytest.mark.parametrize("name", ["uniform", "geometric", "extreme", "random"])
def test_long_strings_round_trip_within_the_entropy_bound(oracle_lib, name):
    rng = np.random.default_rng(hash(name) % 2**32)
    f = tables_256(rng)[name]
    p = f.astype(np.float64) / PTOT
    for n in (0, 1, 7, 150, 1000, 5000):
        s = rng.choice(256, n, p=p).astype(np.uint8)
        data = oracle_lib.rc_encode(s, f)
        junk = rng.integers(0, 256, 8, dtype=np.uint8).tobytes()
        back, _, bad = oracle_lib.rc_decode(data + junk, n, f)
        assert not bad and np.array_equal(back, s)
        c = cost_bits(s, f)
        assert c <= 8 * len(data) <= c + 0.0028 * n + 16


def test_uniform_table_costs_eight_bits_a_symbol(oracle_lib):
    f = tables_256(np.random.default_rng(2))["uniform"]
    rng = np.random.default_rng(3)
    for n in (1, 10, 150, 4000):
        data = oracle_lib.rc_encode(rng.integers(0, 256, n, dtype=np.uint8), f)
        # n bytes of information; the coder loses < 0.0028 bits a symbol to
        # truncation, the flush adds one or two bytes
        assert n <= len(data) <= n + 2 + (0.0028 * n) / 8


def test_normalisation_of_256_counts(oracle_lib):
    rng = np.random.default_rng(4)
    for counts in (np.zeros(256, np.uint32), rng.integers(0, 10**6, 256).astype(np.uint32),
                   np.where(np.arange(256) == 200, 10**7, 0).astype(np.uint32),
                   (rng.random(256) < 0.1).astype(np.uint32) * 5):
        f = oracle_lib.normalize(counts).astype(np.int64)
        assert f.sum() == PTOT and f.min() >= 1
        if counts.sum() == 0:
            assert np.all(f == 128)
            continue
        base = 1 + counts.astype(np.int64) * (PTOT - 256) // int(counts.sum())
        best = int(np.argmax(counts))  # first index of the largest count
        assert np.array_equal(np.delete(f, best), np.delete(base, best))
        assert f[best] == base[best] + PTOT - base.sum()


def small_workload(**kw):
    base = dict(name="anchors", layers=3, tokens=700, channels=70, seed=13, rho=0.85,
                outlier_frac=0.03, chunk_tokens=256, group_tokens=10,
                layer_group_end=(1, 2, 3), layer_step=(0.5, 1.0, 1.5), qualities=(0, 1, 2))
    base.update(kw)
    return synth.Workload(**base)


def numpy_anchors(w, x, inv_a):
    """int anchors [L, groups over all chunks, C] of one [L,T,C] tensor: the first
    token of every group of every chunk, clamp(rint(x * inv_a), -127, 127) in
    binary32."""
    starts = [t0 + g0 for t0 in range(0, w.tokens, w.chunk_tokens)
              for g0 in range(0, min(w.chunk_tokens, w.tokens - t0), w.group_tokens)]
    xs = x[:, starts, :].astype(np.float32)
    a = np.rint(xs * inv_a[:, None, :].astype(np.float32))
    return np.clip(a, -127, 127).astype(np.int64)


def test_anchor_tables_are_the_normalised_anchor_histograms(oracle_lib):
    w = small_workload()
    k, v = synth.gen_kv(w)
    t = oracle_lib.build_tables(oracle_lib.params_for(w, anchor_coding=1), k, v)
    tv = oracle_lib.tables_view(t)
    assert tv.header["version"] == 2 and tv.afreq.shape == (2, w.layers, 256)
    raw = oracle_lib.tables_view(oracle_lib.build_tables(oracle_lib.params_for(w), k, v))
    assert raw.header["version"] == 1 and raw.afreq is None
    # everything else in the tables is the same
    assert np.array_equal(tv.scale_a, raw.scale_a)
    for q in range(3):
        assert np.array_equal(tv.freq[q], raw.freq[q])
    for kv, x in enumerate((k, v)):
        a = numpy_anchors(w, x, tv.inv_a[kv])
        for l in range(w.layers):
            counts = np.bincount(a[l].ravel() + 128, minlength=256).astype(np.uint32)
            assert counts.sum() == a[l].size and counts[0] == 0
            assert np.array_equal(tv.afreq[kv, l], oracle_lib.normalize(counts))


@pytest.mark.parametrize("shape", [dict(), dict(group_tokens=1), dict(group_tokens=64),
                                   dict(tokens=300, chunk_tokens=300, group_tokens=7),
                                   dict(channels=129, tokens=40, chunk_tokens=16)])
def test_coded_blobs_decode_like_raw_blobs(oracle_lib, shape):
    w = small_workload(**shape)
    k, v = synth.gen_kv(w)
    t_raw = oracle_lib.build_tables(oracle_lib.params_for(w), k, v)
    t_cod = oracle_lib.build_tables(oracle_lib.params_for(w, anchor_coding=1), k, v)
    tv = oracle_lib.tables_view(t_cod)
    for q in w.qualities:
        for ch in range(w.n_chunks):
            b_raw = oracle_lib.encode_chunk(t_raw, k, v, ch, q)
            b_cod = oracle_lib.encode_chunk(t_cod, k, v, ch, q)
            h = oracle_lib.parse_blob_header(b_cod)
            assert oracle_lib.parse_blob_header(b_raw)["version"] == 2 and h["version"] == 3
            assert len(b_cod) <= oracle_lib.encode_bound(t_cod, ch)
            outs = []
            for t, b in ((t_raw, b_raw), (t_cod, b_cod)):
                ko, vo = np.zeros_like(k), np.zeros_like(v)
                assert not oracle_lib.decode_blob(t, b, ko, vo)
                outs.append((ko.view(np.uint16), vo.view(np.uint16)))
            assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
            # each anchor stream is the range code of that stream's anchors + 128
            vr, vc = oracle_lib.blob_view(b_raw), oracle_lib.blob_view(b_cod)
            assert vc.anchors is None and np.array_equal(vr.lengths, vc.lengths)
            ng = h["n_groups"]
            for kv in range(2):
                for l in range(w.layers):
                    for c in (0, w.channels // 2, w.channels - 1):
                        f = tv.afreq[kv, l]
                        want = vr.anchors[kv, l, :, c].astype(np.int64) + 128
                        data = oracle_lib.stream_bytes(vc, kv, l, c, anchors=True)
                        got, _, bad = oracle_lib.rc_decode(data, ng, f)
                        assert not bad and np.array_equal(got, want)
                        enc = oracle_lib.rc_encode(want.astype(np.uint8), f)
                        assert vc.anchor_lengths[kv, l, c] == -(-len(enc) // 4)
            # the delta streams are unchanged, at their new place
            for kv, l, c in ((0, 0, 0), (1, w.layers - 1, w.channels - 1)):
                assert (oracle_lib.stream_bytes(vr, kv, l, c)
                        == oracle_lib.stream_bytes(vc, kv, l, c))


def test_coded_anchors_cost_about_their_entropy(oracle_lib):
    """The anchor streams together cost the anchors' cross entropy under the
    tables (within the coder's loss and a flush per stream), which is below the
    8 raw bits on this source; the whole blob shrinks by the difference."""
    w = small_workload(tokens=1536, chunk_tokens=1536, channels=128)
    k, v = synth.gen_kv(w)
    t_cod = oracle_lib.build_tables(oracle_lib.params_for(w, anchor_coding=1), k, v)
    t_raw = oracle_lib.build_tables(oracle_lib.params_for(w), k, v)
    tv = oracle_lib.tables_view(t_cod)
    b_cod = oracle_lib.encode_chunk(t_cod, k, v, 0, 0)
    b_raw = oracle_lib.encode_chunk(t_raw, k, v, 0, 0)
    vc = oracle_lib.blob_view(b_cod)
    vr = oracle_lib.blob_view(b_raw)
    ng = vc.header["n_groups"]
    coded_bits = 32 * int(vc.anchor_lengths.astype(np.int64).sum())
    cross = 0.0
    for kv in range(2):
        for l in range(w.layers):
            s = vr.anchors[kv, l].astype(np.int64) + 128
            cross += cost_bits(s.ravel(), tv.afreq[kv, l])
    n_streams = 2 * w.layers * w.channels
    assert cross <= coded_bits <= cross + 0.0028 * n_streams * ng + n_streams * (16 + 31)
    raw_bits = 8 * 2 * w.layers * ng * w.channels
    assert coded_bits < 0.95 * raw_bits
    saved = len(b_raw) - len(b_cod)
    # raw anchor bytes minus coded anchor words and their lengths and row offsets
    expect = raw_bits // 8 - coded_bits // 8 - 2 * 2 * w.layers * w.channels - 4 * 2 * w.layers
    assert abs(saved - expect) <= 32


def test_coded_blobs_need_their_tables(oracle_lib):
    w = small_workload(tokens=200, chunk_tokens=200)
    k, v = synth.gen_kv(w)
    t_raw = oracle_lib.build_tables(oracle_lib.params_for(w), k, v)
    t_cod = oracle_lib.build_tables(oracle_lib.params_for(w, anchor_coding=1), k, v)
    b_cod = oracle_lib.encode_chunk(t_cod, k, v, 0, 0)
    ko, vo = np.zeros_like(k), np.zeros_like(v)
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.decode_blob(t_raw, b_cod, ko, vo)
    # a coded blob claiming raw anchors (version 2) is refused by its own tables
    forged = bytearray(b_cod)
    forged[4] = 2
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.decode_blob(t_cod, bytes(forged), ko, vo)


def test_anchor_coding_parameter_checks(oracle_lib):
    w = small_workload(tokens=100, chunk_tokens=100)
    k, v = synth.gen_kv(w)
    for bad in (2, -1):
        with pytest.raises(oracle_lib.OracleError):
            oracle_lib.build_tables(oracle_lib.params_for(w, anchor_coding=bad), k, v)
    # channels x tokens must stay below 2^32 so that a layer's anchor counts fit
    p = oracle_lib.make_params(2, 1 << 21, 2048, 1024, 10, (1, 2), (0.5, 1.0), quality_mask=1,
                               anchor_coding=1)
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.build_tables(p, np.zeros((2, 1, 1), np.float16), np.zeros((2, 1, 1), np.float16))
