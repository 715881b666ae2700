"""Pins the oracle's codec end to end: lossless symbols, the reconstruction
error bound, which token is the anchor, the delta grid, the coded length
against the empirical entropy, the coded size against the analytic entropy of
the synthetic source, and the container layout."""
import math

import numpy as np
import pytest
from scipy.stats import norm

import synth

M = 1 << 15


def mk(name="w", **kw):
    base = dict(layers=3, tokens=1000, channels=64, seed=31, rho=0.85, outlier_frac=0.03,
                chunk_tokens=384, group_tokens=10, layer_group_end=(1, 2, 3),
                layer_step=(0.5, 1.0, 1.5), qualities=(0, 1, 2))
    base.update(kw)
    return synth.Workload(name, **base)


def encode_all(o, w, k, v):
    t = o.build_tables(o.params_for(w), k, v)
    blobs = {(ch, q): o.encode_chunk(t, k, v, ch, q) for ch in range(w.n_chunks)
             for q in w.qualities}
    return t, blobs


def ulp16(y):
    y = np.abs(y.astype(np.float64))
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -14)))
    return 2.0 ** (e - 10)


@pytest.fixture(scope="module")
def coded(oracle_lib):
    w = mk()
    k, v = synth.gen_kv(w)
    t, blobs = encode_all(oracle_lib, w, k, v)
    return w, k, v, t, blobs


def test_symbols_roundtrip_losslessly(oracle_lib, coded):
    w, k, v, t, blobs = coded
    for (ch, q), b in blobs.items():
        anchors, syms = oracle_lib.chunk_symbols(t, k, v, ch, q)
        dec, bad = oracle_lib.decode_blob_symbols(t, b)
        assert not bad
        assert np.array_equal(dec, syms)
        assert np.array_equal(oracle_lib.blob_view(b).anchors, anchors)


def test_reconstruction_error_bound(oracle_lib, coded):
    """Deltas: |y-x| <= step/2 (+ rounding); anchors: |y-x| <= scale_a/2 (+ rounding).
    The anchor bound is ~15x tighter than the delta bound here, so it also pins which
    token of every group is the anchor (the group's first)."""
    w, k, v, t, blobs = coded
    tv = oracle_lib.tables_view(t)
    for q in w.qualities:
        ko, vo = np.zeros_like(k), np.zeros_like(v)
        for ch in range(w.n_chunks):
            assert not oracle_lib.decode_blob(t, blobs[(ch, q)], ko, vo)
        for kv, (x, y) in enumerate(((k, ko), (v, vo))):
            xd, yd = x.astype(np.float64), y.astype(np.float64)
            err = np.abs(yd - xd)
            step = tv.step[q][kv].astype(np.float64)[:, None, :]
            sa = tv.scale_a[kv].astype(np.float64)[:, None, :]
            pos = np.arange(w.tokens) % w.chunk_tokens
            is_anchor = (pos % w.group_tokens == 0)[None, :, None]
            slack = 2.0 ** -21 * (np.abs(xd) + 40 * step) + ulp16(y) / 2
            a_err = np.where(is_anchor, err - (sa / 2 + slack), -1)
            assert a_err.max() <= 0
            _, syms = zip(*[oracle_lib.chunk_symbols(t, k, v, ch, q) for ch in range(w.n_chunks)])
            s = np.concatenate([sy[kv] for sy in syms], axis=1).astype(np.int64)
            clipped = (s == 0) | (s == 63)
            d_err = np.where(~is_anchor & ~clipped, err - (step / 2 + sa / 2 + slack), -1)
            assert d_err.max() <= 0


def test_delta_symbols_on_the_step_grid(oracle_lib, coded):
    """symbol - 32 = round((x - anchor) / step), evaluated in binary64 away from ties,
    with the anchor reconstructed from the stored 8-bit code (a wrong sign, step or
    reference token fails this)."""
    w, k, v, t, blobs = coded
    tv = oracle_lib.tables_view(t)
    for ch in range(w.n_chunks):
        t0 = ch * w.chunk_tokens
        for q in w.qualities:
            anchors, syms = oracle_lib.chunk_symbols(t, k, v, ch, q)
            tc = syms.shape[2]
            for kv, x in enumerate((k, v)):
                xs = x[:, t0:t0 + tc, :].astype(np.float64)
                g = np.arange(tc) // w.group_tokens
                ahat = anchors[kv].astype(np.float64)[:, g, :] * tv.scale_a[kv].astype(np.float64)[:, None, :]
                # the anchor code itself: nearest integer to x / scale_a
                is_a = (np.arange(tc) % w.group_tokens) == 0
                ra = xs[:, is_a, :] / tv.scale_a[kv].astype(np.float64)[:, None, :]
                fa = ra - np.floor(ra)
                ok = np.abs(fa - 0.5) > 1e-4
                assert np.array_equal(np.round(ra)[ok], anchors[kv].astype(np.float64)[ok])
                u = (xs - ahat) / tv.step[q][kv].astype(np.float64)[:, None, :]
                want = np.clip(np.round(u), -32, 31) + 32
                frac = np.abs(u - np.floor(u) - 0.5)
                sel = (~is_a)[None, :, None] & (frac > 1e-4)
                assert np.array_equal(syms[kv][sel].astype(np.float64), want[sel])


def test_coded_length_within_entropy_bound(oracle_lib, coded):
    """Payload bits <= 1.01 * sum(-log2 p_emp) + 16 bits per stream, with p_emp the
    empirical symbol frequency of each (kv, quality, layer, channel) over the encoded
    data (all chunks); word padding is reported separately."""
    w, k, v, t, blobs = coded
    _, counts = oracle_lib.build_tables(oracle_lib.params_for(w), k, v, with_counts=True)
    for qi, q in enumerate(w.qualities):
        c = counts[qi].astype(np.float64)
        N = c.sum(axis=-1, keepdims=True)
        with np.errstate(divide="ignore", invalid="ignore"):
            h = np.where(c > 0, -c * np.log2(c / N), 0.0).sum()
        words = sum(int(oracle_lib.blob_view(blobs[(ch, q)]).header["payload_words"])
                    for ch in range(w.n_chunks))
        streams = 2 * w.layers * w.channels * w.n_chunks
        bits = 32 * words - 31 * streams  # at most 31 padding bits per stream
        assert bits <= 1.01 * h + 16 * streams, (q, bits, h)
        assert 32 * words >= h


def analytic_bits_per_delta(rho, h, G=10):
    """Entropy of the delta symbol of an AR(1) source under one table per channel:
    x_t - x_anchor ~ N(0, 2(1-rho^t)) channel variances at distance t, quantised with
    step h channel stds; the table sees the equal mixture over t = 1..G-1."""
    ks = np.arange(-32, 32, dtype=np.float64)
    mix = np.zeros(64)
    for t in range(1, G):
        sd = math.sqrt(2 * (1 - rho ** t)) / h
        hi = norm.cdf((ks + 0.5) / sd)
        lo = norm.cdf((ks - 0.5) / sd)
        hi[-1], lo[0] = 1.0, 0.0
        mix += (hi - lo) / (G - 1)
    p = mix[mix > 0]
    return float(-(p * np.log2(p)).sum())


def test_entropy_matches_the_source_model(oracle_lib):
    """Empirical entropy of the delta symbols and the coded size both agree with the
    closed-form entropy of the synthetic AR(1) source, per layer group and quality."""
    w = mk(tokens=6144, channels=128, chunk_tokens=1536, seed=41)
    k, v = synth.gen_kv(w)
    t, counts = oracle_lib.build_tables(oracle_lib.params_for(w), k, v, with_counts=True)
    for qi, q in enumerate(w.qualities):
        for l in range(3):
            hstep = w.quality_mult[q] * w.layer_step[l]
            want = analytic_bits_per_delta(w.rho, hstep)
            c = counts[qi][:, l].astype(np.float64)
            N = c.sum(axis=-1, keepdims=True)
            with np.errstate(divide="ignore", invalid="ignore"):
                got = np.where(c > 0, -c / N * np.log2(c / N), 0).sum(axis=-1).mean()
            assert abs(got - want) <= 0.015 * want, (q, l, got, want)
    for q in w.qualities:
        words = sum(oracle_lib.blob_view(oracle_lib.encode_chunk(t, k, v, ch, q))
                    .header["payload_words"] for ch in range(w.n_chunks))
        n_sym = 2 * 3 * 128 * sum(tc - -(-tc // 10) for tc in (1536,) * 4)
        want = sum(analytic_bits_per_delta(w.rho, w.quality_mult[q] * s) for s in w.layer_step) / 3
        got = 32 * words / n_sym
        assert want * 0.99 <= got <= want * 1.03, (q, got, want)


def test_reencoding_the_decoded_tensor_is_idempotent(oracle_lib, coded):
    w, k, v, t, blobs = coded
    for q in w.qualities:
        ko, vo = np.zeros_like(k), np.zeros_like(v)
        for ch in range(w.n_chunks):
            oracle_lib.decode_blob(t, blobs[(ch, q)], ko, vo)
        for ch in range(w.n_chunks):
            assert oracle_lib.encode_chunk(t, ko, vo, ch, q) == blobs[(ch, q)]


def test_blob_layout(oracle_lib, coded):
    w, k, v, t, blobs = coded
    tid = oracle_lib.tables_id(t)
    for (ch, q), b in blobs.items():
        bv = oracle_lib.blob_view(b)
        h = bv.header
        t0, tc, ng = oracle_lib.chunk_geometry(t, ch)
        assert h["magic"] == b"CGK1" and h["version"] == 2 and h["prob_bits"] == 15
        assert (h["token_offset"], h["chunk_tokens"], h["n_groups"]) == (t0, tc, ng)
        assert h["quality"] == q and h["tables_id"] == tid
        lens = bv.lengths.astype(np.int64)
        assert lens.sum() == h["payload_words"]
        rows = np.concatenate([[0], np.cumsum(lens.sum(axis=-1).ravel())[:-1]])
        assert np.array_equal(bv.row_offset.ravel(), rows)
        assert len(b) % 16 == 0 and len(bv.tail) >= 16 and not any(bv.tail)
        assert bv.payload_offset % 16 == 0
        assert len(b) <= oracle_lib.encode_bound(t, ch)


def test_payload_block_layout(oracle_lib, coded):
    """The payload layout of a block of streams, on a hand-made block (lengths
    5, 9, 4, 8 words: one whole unit each, m = 1): unit 0 of every stream,
    stream after stream, then the rest of each stream in stream order; and on
    every row of the coded blobs: the streams' words cover the row's payload
    words exactly once (nothing padded, nothing shared), in blocks of 64
    streams in channel order."""
    lens = np.array([5, 9, 4, 8], np.uint16)
    got = [list(oracle_lib.stream_word_offsets(lens, c)) for c in range(4)]
    assert got == [[0, 1, 2, 3, 16], [4, 5, 6, 7, 17, 18, 19, 20, 21],
                   [8, 9, 10, 11], [12, 13, 14, 15, 22, 23, 24, 25]]
    lens2 = np.array([3, 12, 7], np.uint16)  # a stream shorter than a unit: m = 0
    assert [list(oracle_lib.stream_word_offsets(lens2, c)) for c in range(3)] == [
        [0, 1, 2], list(range(3, 15)), list(range(15, 22))]
    w, k, v, t, blobs = coded
    for (ch, q), b in list(blobs.items())[:3]:
        bv = oracle_lib.blob_view(b)
        for kv in range(2):
            for l in range(w.layers):
                at = np.concatenate([oracle_lib.stream_word_offsets(bv.lengths[kv, l], c)
                                     for c in range(w.channels)])
                assert np.array_equal(np.sort(at), np.arange(int(bv.lengths[kv, l].sum())))
                for c0 in range(0, w.channels, 64):  # a block's words are its own
                    base = int(bv.lengths[kv, l, :c0].astype(np.int64).sum())
                    blk = np.concatenate([oracle_lib.stream_word_offsets(bv.lengths[kv, l], c)
                                          for c in range(c0, min(c0 + 64, w.channels))])
                    assert blk.min() == base and blk.max() == base + len(blk) - 1


def test_single_stream_api_matches_blobs(oracle_lib, coded):
    """The per-stream entry points (used for sampled checks at full size) agree with
    the whole-chunk ones, and decoding ignores what follows a stream."""
    w, k, v, t, blobs = coded
    rng = np.random.default_rng(3)
    for (ch, q), b in list(blobs.items())[::2]:
        bv = oracle_lib.blob_view(b)
        t0, tc, ng = oracle_lib.chunk_geometry(t, ch)
        ko, vo = np.zeros_like(k), np.zeros_like(v)
        oracle_lib.decode_blob(t, b, ko, vo)
        for _ in range(12):
            kv, l, c = int(rng.integers(2)), int(rng.integers(w.layers)), int(rng.integers(w.channels))
            x = (k, v)[kv][l, t0:t0 + tc, c]
            anchors, data = oracle_lib.stream_encode(t, kv, l, c, q, x)
            assert np.array_equal(anchors, bv.anchors[kv, l, :, c])
            n = int(bv.lengths[kv, l, c])
            full = oracle_lib.stream_bytes(bv, kv, l, c)
            assert data == full[: 4 * n]
            want = (ko, vo)[kv][l, t0:t0 + tc, c]
            for tail in (full[4 * n:], b"", rng.integers(0, 256, 16, dtype=np.uint8).tobytes()):
                y, bad = oracle_lib.stream_decode(t, kv, l, c, q, anchors, tc, data + tail)
                assert not bad and np.array_equal(y.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("shape", [
    dict(tokens=1, chunk_tokens=1, group_tokens=1, channels=3),          # one anchor only
    dict(tokens=37, chunk_tokens=16, group_tokens=5, channels=7),        # ragged chunk and group
    dict(tokens=23, chunk_tokens=23, group_tokens=1, channels=5),        # all anchors, empty streams
    dict(tokens=50, chunk_tokens=21, group_tokens=10, channels=1),       # 1-token last group
])
def test_edge_geometries(oracle_lib, shape):
    w = mk(layers=2, layer_group_end=(1, 2), layer_step=(0.5, 1.5), **shape)
    k, v = synth.gen_kv(w)
    t, blobs = encode_all(oracle_lib, w, k, v)
    for q in w.qualities:
        ko, vo = np.zeros_like(k), np.zeros_like(v)
        for ch in range(w.n_chunks):
            b = blobs[(ch, q)]
            assert not oracle_lib.decode_blob(t, b, ko, vo)
            dec, _ = oracle_lib.decode_blob_symbols(t, b)
            assert np.array_equal(dec, oracle_lib.chunk_symbols(t, k, v, ch, q)[1])
        assert np.all(np.isfinite(ko.astype(np.float32)))
        if shape["group_tokens"] == 1:
            assert all(oracle_lib.blob_view(blobs[(ch, q)]).header["payload_words"] == 0
                       for ch in range(w.n_chunks))


def test_degenerate_channels(oracle_lib):
    w = mk(layers=1, tokens=64, channels=4, chunk_tokens=64, layer_group_end=(1,),
           layer_step=(0.5,), qualities=(0,))
    k = np.zeros((1, 64, 4), np.float16)
    v = np.zeros((1, 64, 4), np.float16)
    k[0, :, 1] = 3.25                        # constant: std reads as 1
    k[0, :, 2] = np.float16(-65504)          # extreme constant
    k[0, ::7, 3] = np.float16(1e-7)          # sparse subnormals
    t, blobs = encode_all(oracle_lib, w, k, v)
    tv = oracle_lib.tables_view(t)
    assert tv.scale_a[1, 0, 0] == 1.0 and tv.step[0][0, 0, 1] == 0.5
    ko, vo = np.zeros_like(k), np.zeros_like(v)
    assert not oracle_lib.decode_blob(t, blobs[(0, 0)], ko, vo)
    assert np.array_equal(vo, v) and np.array_equal(ko[..., :3], k[..., :3])
    assert np.all(np.abs(ko[..., 3].astype(np.float64) - k[..., 3]) <= tv.step[0][0, 0, 3])


def test_corrupt_payload_is_flagged_not_crashing(oracle_lib, coded):
    w, k, v, t, blobs = coded
    b = bytearray(blobs[(0, 0)])
    bv = oracle_lib.blob_view(bytes(b))
    # lengths that no longer add up to the row offsets are detected
    off_len = 64 + 8 * w.layers + 2 * w.layers * bv.header["n_groups"] * w.channels
    b[off_len] ^= 0x01
    ko, vo = np.zeros_like(k), np.zeros_like(v)
    assert oracle_lib.decode_blob(t, bytes(b), ko, vo)
    # a blob made for other tables is refused
    t2 = bytearray(t)
    t2[200] ^= 1
    with pytest.raises(oracle_lib.OracleError) as e:
        oracle_lib.decode_blob(bytes(t2), blobs[(0, 0)], ko, vo)
    assert e.value.code == -6


def test_nonfinite_input_is_not_encoded(oracle_lib, coded):
    w, k, v, t, blobs = coded
    k2 = k.copy()
    k2[1, 500, 3] = np.inf
    with pytest.raises(oracle_lib.OracleError) as e:
        oracle_lib.encode_chunk(t, k2, v, 1, 0)
    assert e.value.code == -1
    oracle_lib.encode_chunk(t, k2, v, 0, 0)  # other chunks are unaffected
