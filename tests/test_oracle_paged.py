"""Pins the oracle's paged decode (decode_blob_paged) against the plain decode,
which the codec tests pin: pages in context order reproduce the plain [L, T, C]
tensor (so the layout is layer, page, row, channel and token t sits in row
t mod P of block t div P); relabelling the pages permutes the pool the same way;
pages no block names keep what they held; an entry outside the pool is reported
and only its block's rows are missing; the chunks of a context write disjoint
rows, so their order does not matter; and one page larger than the context is
the plain tensor itself."""
import numpy as np
import pytest

import synth

FILL = np.uint16(0x7E5A)  # a NaN pattern the codec never writes


def mk(**kw):
    base = dict(layers=3, tokens=1000, channels=130, seed=41, rho=0.85, outlier_frac=0.03,
                chunk_tokens=384, group_tokens=10, layer_group_end=(1, 2, 3),
                layer_step=(0.5, 1.0, 1.5), qualities=(0, 1, 2))
    base.update(kw)
    return synth.Workload("paged", **base)


@pytest.fixture(scope="module")
def coded(oracle_lib):
    o = oracle_lib
    w = mk()
    k, v = synth.gen_kv(w)
    t = o.build_tables(o.params_for(w), k, v)
    blobs = [o.encode_chunk(t, k, v, ch, ch % 3) for ch in range(w.n_chunks)]
    L, T, Cc = k.shape
    kd = np.zeros((L, T, Cc), np.float16)
    vd = np.zeros((L, T, Cc), np.float16)
    for b in blobs:
        assert not o.decode_blob(t, b, kd, vd)
    return o, w, t, blobs, kd, vd


def pools(L, n_pages, P, Cc):
    k = np.full((L, n_pages, P, Cc), FILL, np.uint16).view(np.float16)
    v = np.full((L, n_pages, P, Cc), FILL, np.uint16).view(np.float16)
    return k, v


def paged(o, t, blobs, n_pages, P, table, order=None):
    h = o.parse_blob_header(blobs[0])
    k, v = pools(h["layers"], n_pages, P, h["channels"])
    flags = []
    for i in (order if order is not None else range(len(blobs))):
        flags.append(o.decode_blob_paged(t, blobs[i], k, v, P, np.asarray(table, np.int32)))
    return k, v, flags


def bits(a):
    return a.view(np.uint16)


@pytest.mark.parametrize("P", [1, 8, 16, 1000])
def test_pages_in_order_are_the_plain_tensor(coded, P):
    o, w, t, blobs, kd, vd = coded
    L, T, Cc = kd.shape
    nb = -(-T // P)
    k, v, flags = paged(o, t, blobs, nb, P, np.arange(nb))
    assert all(f == (False, False) for f in flags)
    flat_k = bits(k).reshape(L, nb * P, Cc)
    flat_v = bits(v).reshape(L, nb * P, Cc)
    assert np.array_equal(flat_k[:, :T], bits(kd)) and np.array_equal(flat_v[:, :T], bits(vd))
    # rows past the context in the last page are not touched
    assert (flat_k[:, T:] == FILL).all() and (flat_v[:, T:] == FILL).all()


@pytest.mark.parametrize("P", [4, 16])
def test_relabelled_pages_permute_the_pool(coded, P):
    o, w, t, blobs, kd, vd = coded
    T = kd.shape[1]
    nb = -(-T // P)
    spare = 7
    perm = np.random.default_rng(5).permutation(nb + spare)[:nb]
    k0, v0, _ = paged(o, t, blobs, nb, P, np.arange(nb))
    k1, v1, flags = paged(o, t, blobs, nb + spare, P, perm)
    assert all(f == (False, False) for f in flags)
    assert np.array_equal(bits(k1)[:, perm], bits(k0)) and np.array_equal(bits(v1)[:, perm], bits(v0))
    unnamed = np.setdiff1d(np.arange(nb + spare), perm)
    assert unnamed.size == spare
    assert (bits(k1)[:, unnamed] == FILL).all() and (bits(v1)[:, unnamed] == FILL).all()


def test_bad_entries_are_reported_and_skipped(coded):
    o, w, t, blobs, kd, vd = coded
    T = kd.shape[1]
    P = 16
    nb = -(-T // P)
    good = np.arange(nb) + 2          # pages 0 and 1 stay spare
    bad = good.copy()
    bad[3] = nb + 2                   # one past the pool
    bad[40] = -1
    kg, vg, _ = paged(o, t, blobs, nb + 2, P, good)
    kb, vb, flags = paged(o, t, blobs, nb + 2, P, bad)
    # block 3 lies in chunk 0, block 40 (tokens 640..655) in chunk 1
    assert [f[1] for f in flags] == [True, True, False]
    assert not any(f[0] for f in flags)
    for pg in (good[3], good[40]):
        assert (bits(kb)[:, pg] == FILL).all() and (bits(vb)[:, pg] == FILL).all()
    keep = np.setdiff1d(np.arange(nb + 2), [good[3], good[40]])
    assert np.array_equal(bits(kb)[:, keep], bits(kg)[:, keep])
    assert np.array_equal(bits(vb)[:, keep], bits(vg)[:, keep])


def test_chunk_order_does_not_matter(coded):
    o, w, t, blobs, kd, vd = coded
    T = kd.shape[1]
    P = 8
    nb = -(-T // P)
    table = np.random.default_rng(9).permutation(nb)
    ka, va, _ = paged(o, t, blobs, nb, P, table)
    kb, vb, _ = paged(o, t, blobs, nb, P, table, order=[2, 0, 1])
    assert np.array_equal(bits(ka), bits(kb)) and np.array_equal(bits(va), bits(vb))


def test_one_page_larger_than_the_context(coded):
    o, w, t, blobs, kd, vd = coded
    T = kd.shape[1]
    k, v, _ = paged(o, t, blobs, 2, 1024, [1])
    assert np.array_equal(bits(k)[:, 1, :T], bits(kd)) and np.array_equal(bits(v)[:, 1, :T], bits(vd))
    assert (bits(k)[:, 0] == FILL).all() and (bits(k)[:, 1, T:] == FILL).all()
