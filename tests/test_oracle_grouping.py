"""Pins of the oracle's pooled table groupings (what per-(layer, channel)
symbol statistics are worth, CacheGen blog section 1): structure, the case
where pooling changes nothing, and the information-theoretic order of the coded
sizes.  CPU only."""
import numpy as np
import pytest

import oracle
import synth

W = synth.workload("mistral7b_9k", layers=4, tokens=300, channels=130, chunk_tokens=128,
                   layer_group_end=(1, 2, 4))


@pytest.fixture(scope="module")
def kv():
    return synth.gen_kv(W)


def tables(k, v, grouping, w=W):
    return oracle.build_tables_grouped(oracle.params_for(w), k, v, grouping, threads=4)


def test_per_layer_and_channel_is_the_plain_build(kv):
    k, v = kv
    assert tables(k, v, oracle.GROUP_LAYER_CHANNEL) == oracle.build_tables(
        oracle.params_for(W), k, v, threads=4)


@pytest.mark.parametrize("grouping", [oracle.GROUP_LAYER, oracle.GROUP_CHANNEL,
                                      oracle.GROUP_GLOBAL])
def test_group_members_share_one_table_and_keep_their_scales(kv, grouping):
    k, v = kv
    t0 = oracle.tables_view(tables(k, v, oracle.GROUP_LAYER_CHANNEL))
    tg = oracle.tables_view(tables(k, v, grouping))
    assert np.array_equal(t0.scale_a, tg.scale_a) and np.array_equal(t0.inv_a, tg.inv_a)
    for q in W.qualities:
        assert np.array_equal(t0.step[q], tg.step[q])
        f = tg.freq[q]                         # [2, L, C, 64]
        assert (f.sum(axis=-1) == 1 << 15).all() and f.min() >= 1
        if grouping == oracle.GROUP_LAYER:
            assert (f == f[:, :, :1]).all()
        elif grouping == oracle.GROUP_CHANNEL:
            assert (f == f[:, :1]).all()
        else:
            assert (f == f[:, :1, :1]).all()
        assert not np.array_equal(f, t0.freq[q])


def test_pooling_identical_members_changes_nothing():
    # every channel a copy of channel 0: pooling over channels sums equal counts,
    # and 1 + floor(n c s / (n N)) = 1 + floor(c s / N)
    w = synth.workload("tiny", channels=16)
    k, v = synth.gen_kv(w)
    k = np.ascontiguousarray(np.repeat(k[:, :, :1], 16, axis=2))
    v = np.ascontiguousarray(np.repeat(v[:, :, :1], 16, axis=2))
    assert tables(k, v, oracle.GROUP_LAYER, w) == tables(k, v, oracle.GROUP_LAYER_CHANNEL, w)
    # every layer a copy of layer 0 (one layer group, so equal steps)
    k = np.ascontiguousarray(np.repeat(k[:1], 2, axis=0))
    v = np.ascontiguousarray(np.repeat(v[:1], 2, axis=0))
    assert tables(k, v, oracle.GROUP_CHANNEL, w) == tables(k, v, oracle.GROUP_LAYER_CHANNEL, w)
    assert tables(k, v, oracle.GROUP_GLOBAL, w) == tables(k, v, oracle.GROUP_LAYER_CHANNEL, w)


def test_finer_statistics_never_code_longer(kv):
    # the empirical distribution of a stream's own symbols minimises its cross
    # entropy, so coding with pooled tables costs at least as much, up to the
    # tables' rounding to 15-bit frequencies
    k, v = kv
    size = {}
    for g in (oracle.GROUP_LAYER_CHANNEL, oracle.GROUP_LAYER, oracle.GROUP_CHANNEL,
              oracle.GROUP_GLOBAL):
        t = tables(k, v, g)
        size[g] = sum(len(oracle.encode_chunk(t, k, v, ch, q, threads=4))
                      for ch in range(W.n_chunks) for q in W.qualities)
    fine = size[oracle.GROUP_LAYER_CHANNEL]
    for g in (oracle.GROUP_LAYER, oracle.GROUP_CHANNEL, oracle.GROUP_GLOBAL):
        assert fine <= size[g] * 1.002, size
    assert size[oracle.GROUP_LAYER] <= size[oracle.GROUP_GLOBAL] * 1.002
    assert size[oracle.GROUP_CHANNEL] <= size[oracle.GROUP_GLOBAL] * 1.002


def test_a_pooled_count_must_fit_32_bits():
    c = np.full((1, 2, 3, 4, 64), 0x7FFFFFFF, np.uint32)
    with pytest.raises(ValueError):
        oracle.pool_counts(c, oracle.GROUP_LAYER)
    assert oracle.pool_counts(c[:, :, :, :1], oracle.GROUP_LAYER).max() == 0x7FFFFFFF
    with pytest.raises(ValueError):
        oracle.pool_counts(c, 7)
