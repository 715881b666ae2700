"""GPU parity: the HIP path (through the C ABI) against the oracle on the same
seeded inputs.  Integer and byte results (tables, blobs) must be identical; the
fp16 reconstruction must be bit-identical (within 1 ulp is the stated bar, 0
is what the shared binary32 op sequence gives)."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def run_all(w, check_cross=True):
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    import kv_cache_compression_anchor_amd as cg
    gt = cg.cg_tables_serialize(tab)
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    assert gt == ot, ("tables differ", gu.first_difference(gt, ot))
    assert tab.id == oracle.tables_id(ot)
    for ch in range(w.n_chunks):
        for q in w.qualities:
            dblob, gb = gu.gpu_encode(tab, kd, vd, ch, q)
            ob = oracle.encode_chunk(ot, k, v, ch, q)
            assert gb == ob, ("blob differs", ch, q, gu.first_difference(gb, ob))
            kg, vg, st = gu.gpu_decode(tab, [dblob], k.shape)
            ko, vo, bad = gu.oracle_decode(ot, [ob], k.shape)
            assert st == 0 and not bad
            assert gu.same_bits(kg, ko) and gu.same_bits(vg, vo), ("decode differs", ch, q)
    return k, v, kd, vd, tab, ot


def test_tiny_workload():
    run_all(synth.workload("tiny"))


def test_multi_chunk_ragged_three_qualities():
    # 3 chunks (last one ragged), ragged last group, channels not a multiple of 64
    run_all(gu.workload())


@pytest.mark.parametrize("shape", [
    dict(tokens=1, chunk_tokens=1, group_tokens=1, channels=3),
    dict(tokens=37, chunk_tokens=16, group_tokens=5, channels=7),
    dict(tokens=23, chunk_tokens=23, group_tokens=1, channels=65),
    dict(tokens=50, chunk_tokens=21, group_tokens=10, channels=1),
    dict(tokens=300, chunk_tokens=300, group_tokens=300, channels=130),
    dict(tokens=129, chunk_tokens=64, group_tokens=3, channels=64),
])
def test_edge_geometries(shape):
    run_all(gu.workload(layers=2, layer_group_end=(1, 2), layer_step=(0.5, 1.5), **shape))


def test_selection_of_mixed_qualities_in_one_call():
    """Several chunks at different qualities decoded by one cg_decode_async call
    (chunks of one quality share a workgroup's LDS tables)."""
    w = gu.workload(tokens=2000, chunk_tokens=256, channels=192)
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    import kv_cache_compression_anchor_amd as cg
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    assert cg.cg_tables_serialize(tab) == ot
    sel = [(ch, (ch * 7) % 3) for ch in range(w.n_chunks)]
    dblobs, hblobs = zip(*[gu.gpu_encode(tab, kd, vd, ch, q) for ch, q in sel])
    obs = [oracle.encode_chunk(ot, k, v, ch, q) for ch, q in sel]
    assert list(hblobs) == obs
    kg, vg, st = gu.gpu_decode(tab, list(dblobs), k.shape)
    ko, vo, bad = gu.oracle_decode(ot, obs, k.shape)
    assert st == 0 and not bad
    assert gu.same_bits(kg, ko) and gu.same_bits(vg, vo)
    # and the synchronous entry point gives the same
    t = gu.torch()
    k2 = t.zeros_like(kd)
    v2 = t.zeros_like(vd)
    cg.cg_decode(tab, list(dblobs), k2, v2)
    assert gu.same_bits(k2.cpu().numpy(), ko) and gu.same_bits(v2.cpu().numpy(), vo)


def test_cross_decoding_both_ways():
    w = gu.workload(tokens=700, channels=70, seed=9)
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    import kv_cache_compression_anchor_amd as cg
    # tables made by the oracle, uploaded: the GPU decodes oracle blobs
    tab2 = cg.cg_tables_deserialize(ot)
    assert tab2.id == tab.id
    for q in w.qualities:
        obs = [oracle.encode_chunk(ot, k, v, ch, q) for ch in range(w.n_chunks)]
        dev = [gu.to_dev(np.frombuffer(b, np.uint8).copy()) for b in obs]
        kg, vg, st = gu.gpu_decode(tab2, dev, k.shape)
        ko, vo, _ = gu.oracle_decode(ot, obs, k.shape)
        assert st == 0 and gu.same_bits(kg, ko) and gu.same_bits(vg, vo)
        # and the GPU encodes exactly the oracle's blobs, which the oracle decodes
        gbs = [gu.gpu_encode(tab, kd, vd, ch, q)[1] for ch in range(w.n_chunks)]
        assert gbs == obs


@pytest.mark.parametrize("group_tokens", [10, 7])
def test_costly_symbols_drain_the_word_ring(group_tokens):
    """Tables built from one K/V pair, data from another whose deltas all hit
    the clipped extremes, each of which the tables give a tiny probability:
    about 15 bits per symbol, more than the decoder's per-group word fetches
    supply, so its direct-load refill runs (group size 10 takes the unrolled
    path, 7 the generic one)."""
    w = gu.workload(layers=2, tokens=900, channels=70, chunk_tokens=450,
                    group_tokens=group_tokens, layer_group_end=(1, 2), layer_step=(0.5, 1.0),
                    qualities=(0, 2))
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    sign = np.where(np.arange(w.tokens) % 2 == 0, 1.0, -1.0)[None, :, None]
    k2 = (k.astype(np.float32) + 3000.0 * sign).astype(np.float16)
    v2 = (v.astype(np.float32) - 3000.0 * sign).astype(np.float16)
    kd2, vd2 = gu.to_dev(k2), gu.to_dev(v2)
    import kv_cache_compression_anchor_amd as cg
    for ch in range(w.n_chunks):
        for q in w.qualities:
            out = gu.torch().empty(cg.cg_encode_bound(tab, ch), dtype=gu.torch().uint8,
                                   device="cuda")
            n = cg.cg_encode(tab, kd2, vd2, ch, q, out)
            gb = out[:n].cpu().numpy().tobytes()
            ob = oracle.encode_chunk(ot, k2, v2, ch, q)
            assert gb == ob, ("blob differs", ch, q, gu.first_difference(gb, ob))
            bv = oracle.blob_view(ob)
            tc = oracle.parse_blob_header(ob)["chunk_tokens"]
            assert bv.lengths.mean() * 32 > 12 * tc, "streams are not costly enough"
            kg, vg, st = gu.gpu_decode(tab, [out[:n]], k.shape)
            ko, vo, bad = gu.oracle_decode(ot, [ob], k.shape)
            assert st == 0 and not bad
            assert gu.same_bits(kg, ko) and gu.same_bits(vg, vo), ("decode differs", ch, q)
    # both chunks of a quality in one call: a workgroup of two chunks, the
    # LDS-window decoder, whose ring these streams also outrun
    for q in w.qualities:
        dev = [gu.gpu_encode(tab, kd2, vd2, ch, q)[0] for ch in range(w.n_chunks)]
        obs = [oracle.encode_chunk(ot, k2, v2, ch, q) for ch in range(w.n_chunks)]
        kg, vg, st = gu.gpu_decode(tab, dev, k.shape)
        ko, vo, bad = gu.oracle_decode(ot, obs, k.shape)
        assert st == 0 and not bad
        assert gu.same_bits(kg, ko) and gu.same_bits(vg, vo), ("window decode differs", q)


@pytest.mark.parametrize("group_tokens", [1, 2, 3, 4, 7, 10, 13])
def test_several_chunks_of_a_quality_every_group_size(group_tokens):
    """All chunks of a quality decoded by one call (workgroups of several
    chunks: the LDS-window decoder), for group sizes whose deltas split into
    windows of 1, 2 and 3 symbols, a ragged last chunk and last group, and
    channels that end inside a 64-channel block."""
    w = gu.workload(layers=2, tokens=700, channels=100, chunk_tokens=128,
                    group_tokens=group_tokens, layer_group_end=(1, 2), layer_step=(0.5, 1.5),
                    qualities=(0, 2))
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    import kv_cache_compression_anchor_amd as cg
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    assert cg.cg_tables_serialize(tab) == ot
    for q in w.qualities:
        dev, host = zip(*[gu.gpu_encode(tab, kd, vd, ch, q) for ch in range(w.n_chunks)])
        obs = [oracle.encode_chunk(ot, k, v, ch, q) for ch in range(w.n_chunks)]
        assert list(host) == obs, ("blob differs", group_tokens, q)
        kg, vg, st = gu.gpu_decode(tab, list(dev), k.shape)
        ko, vo, bad = gu.oracle_decode(ot, obs, k.shape)
        assert st == 0 and not bad
        assert gu.same_bits(kg, ko) and gu.same_bits(vg, vo), ("decode differs", group_tokens, q)


def test_degenerate_channels():
    w = gu.workload(layers=1, tokens=64, channels=6, chunk_tokens=64, layer_group_end=(1,),
                    layer_step=(0.5,), qualities=(0,))
    k = np.zeros((1, 64, 6), np.float16)
    v = np.zeros((1, 64, 6), np.float16)
    k[0, :, 1] = 3.25
    k[0, :, 2] = np.float16(-65504)
    k[0, ::7, 3] = np.float16(1e-7)
    k[0, :, 4] = np.float16(6e-8) * np.arange(64) % 3
    k[0, :, 5] = np.float16(60000) * (np.arange(64) % 2)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    import kv_cache_compression_anchor_amd as cg
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    assert cg.cg_tables_serialize(tab) == ot
    dblob, gb = gu.gpu_encode(tab, kd, vd, 0, 0)
    ob = oracle.encode_chunk(ot, k, v, 0, 0)
    assert gb == ob
    kg, vg, st = gu.gpu_decode(tab, [dblob], k.shape)
    ko, vo, _ = gu.oracle_decode(ot, [ob], k.shape)
    assert st == 0 and gu.same_bits(kg, ko) and gu.same_bits(vg, vo)


def test_nonfinite_input_is_rejected():
    import kv_cache_compression_anchor_amd as cg
    w = gu.workload(layers=1, tokens=40, channels=8, chunk_tokens=40, layer_group_end=(1,),
                    layer_step=(0.5,), qualities=(0,))
    k, v = synth.gen_kv(w)
    v[0, 5, 5] = np.nan
    with pytest.raises(cg.CgError) as e:
        gu.gpu_tables(w, gu.to_dev(k), gu.to_dev(v))
    assert e.value.code == cg.CG_E_INVAL


def test_nonfinite_input_is_not_encoded():
    import kv_cache_compression_anchor_amd as cg
    w = gu.workload(layers=1, tokens=80, channels=8, chunk_tokens=40, layer_group_end=(1,),
                    layer_step=(0.5,), qualities=(0,))
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    kd[0, 45, 2] = float("inf")
    gu.gpu_encode(tab, kd, vd, 0, 0)
    with pytest.raises(cg.CgError) as e:
        gu.gpu_encode(tab, kd, vd, 1, 0)
    assert e.value.code == cg.CG_E_INVAL


def test_encode_batch_matches_single_encodes_and_oracle():
    """cg_encode_batch over more blobs than one launch holds (several launches,
    shared scratch slots) gives the same bytes as cg_encode and the oracle."""
    import kv_cache_compression_anchor_amd as cg
    w = gu.workload(tokens=2600, chunk_tokens=400, channels=130, seed=12)
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    t = gu.torch()
    jobs = [(ch, q) for ch in range(w.n_chunks) for q in w.qualities]  # 7 x 3 = 21 blobs
    assert len(jobs) > 16
    outs = [t.empty(cg.cg_encode_bound(tab, ch), dtype=t.uint8, device="cuda") for ch, _ in jobs]
    sizes = cg.cg_encode_batch(tab, kd, vd, [j[0] for j in jobs], [j[1] for j in jobs], outs)
    for (ch, q), o, n in zip(jobs, outs, sizes):
        b = o[:n].cpu().numpy().tobytes()
        assert b == oracle.encode_chunk(ot, k, v, ch, q), (ch, q)
        assert b == gu.gpu_encode(tab, kd, vd, ch, q)[1]


def test_encode_batch_reports_capacity_per_blob():
    import kv_cache_compression_anchor_amd as cg
    w = gu.workload(tokens=300, chunk_tokens=150, channels=64, qualities=(0,),
                    layer_group_end=(1, 2, 3))
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    t = gu.torch()
    small = t.empty(4096, dtype=t.uint8, device="cuda")   # fixed part fits, payload does not
    big = t.empty(cg.cg_encode_bound(tab, 1), dtype=t.uint8, device="cuda")
    with pytest.raises(cg.CgError) as e:
        cg.cg_encode_batch(tab, kd, vd, [0, 1], [0, 0], [small, big])
    assert e.value.code == cg.CG_E_CAPACITY
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    n = cg.cg_encode(tab, kd, vd, 1, 0, big)
    assert big[:n].cpu().numpy().tobytes() == oracle.encode_chunk(ot, k, v, 1, 0)


def test_streamed_decode_reuses_staging_slots():
    """cg_decode_streamed with a staging buffer of two slots for five chunks:
    every slot is reused, copies and decodes are ordered by events, and the
    result equals the one-call decode from device memory."""
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    w = gu.workload(tokens=1800, chunk_tokens=384, channels=96, seed=21)
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    sel = [(ch, (ch + 1) % 3) for ch in range(w.n_chunks)]
    dev = [gu.gpu_encode(tab, kd, vd, ch, q)[0] for ch, q in sel]
    host = [b.cpu().pin_memory() for b in dev]
    infos = [cg.cg_chunk_info_parse(h[:64]) for h in host]
    slot = max((b.numel() + 255) // 256 * 256 for b in dev)
    ko = t.zeros_like(kd)
    vo = t.zeros_like(vd)
    st = t.zeros(1, dtype=t.int32, device="cuda")
    stage = t.empty(2 * slot, dtype=t.uint8, device="cuda")
    cs, ks = t.cuda.Stream(), t.cuda.Stream()
    cg.cg_decode_streamed(tab, host, infos, ko, vo, stage, st, cs, ks)
    ks.synchronize()
    k2, v2, st2 = gu.gpu_decode(tab, dev, k.shape)
    assert int(st.item()) == 0 and st2 == 0
    assert gu.same_bits(ko.cpu().numpy(), k2) and gu.same_bits(vo.cpu().numpy(), v2)
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    rk, rv, _ = gu.oracle_decode(ot, [oracle.encode_chunk(ot, k, v, ch, q) for ch, q in sel],
                                 k.shape)
    assert gu.same_bits(k2, rk) and gu.same_bits(v2, rv)
    with pytest.raises(cg.CgError) as e:
        cg.cg_decode_streamed(tab, host, infos, ko, vo, stage[: slot // 2], st, cs, ks)
    assert e.value.code == cg.CG_E_CAPACITY


def test_decode_rejects_mismatched_blobs():
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    w = gu.workload(layers=1, tokens=200, channels=64, chunk_tokens=100, layer_group_end=(1,),
                    layer_step=(0.5,), qualities=(0,))
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    blob = gu.gpu_encode(tab, kd, vd, 0, 0)[0]
    v2 = v.copy()
    v2[0, 0, 0] += np.float16(1.0)
    other = gu.gpu_tables(w, kd, gu.to_dev(v2))          # different tables id
    ko, vo = t.zeros_like(kd), t.zeros_like(vd)
    with pytest.raises(cg.CgError) as e:
        cg.cg_decode(other, [blob], ko, vo)
    assert e.value.code == cg.CG_E_MISMATCH
    info = cg.cg_chunk_info_parse(blob[:64].cpu())
    info.quality = 2                                       # not in the tables
    st = t.zeros(1, dtype=t.int32, device="cuda")
    with pytest.raises(cg.CgError) as e:
        cg.cg_decode_async(tab, [blob], [info], ko, vo, st)
    assert e.value.code == cg.CG_E_MISMATCH


def test_corrupt_payload_is_flagged_without_fault():
    """Flipped payload bytes and wrong stream lengths never fault (reads are
    bounded by the blob); impossible states set the status word."""
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    w = gu.workload(layers=2, tokens=300, channels=128, chunk_tokens=300,
                    layer_group_end=(1, 2), layer_step=(0.5, 1.0), qualities=(0,))
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    blob, hb = gu.gpu_encode(tab, kd, vd, 0, 0)
    bv = oracle.blob_view(hb)
    flagged = 0
    rng = np.random.default_rng(1)
    for trial in range(6):
        bad = blob.clone()
        if trial % 2:
            # lengths beyond the payload: streams start past its end
            off_len = 64 + 8 * w.layers + 2 * w.layers * bv.header["n_groups"] * w.channels
            bad[off_len: off_len + 2] = t.tensor([0xFF, 0xFF], dtype=t.uint8)
        else:
            pos = bv.payload_offset + rng.integers(0, 4 * bv.header["payload_words"], 64)
            bad[t.as_tensor(pos, device="cuda")] ^= 0xA5
        ko, vo = t.zeros_like(kd), t.zeros_like(vd)
        st = t.zeros(1, dtype=t.int32, device="cuda")
        info = cg.cg_chunk_info_parse(bad[:64].cpu())
        cg.cg_decode_async(tab, [bad], [info], ko, vo, st)
        t.cuda.synchronize()
        flagged += int(st.item()) != 0
        if trial % 2:
            assert int(st.item()) != 0
    assert flagged >= 3


def plant_symbols(x, tv, kv, l, c, q, syms, G):
    """Overwrite channel c of layer l so that its delta symbols at quality q are
    `syms` (anchors quantise to 0, each delta token is (s - 32) * step)."""
    step = float(tv.step[q][kv, l, c])
    T = x.shape[1]
    d = iter(syms)
    for t in range(T):
        if t % G == 0:
            x[l, t, c] = 0.0
        else:
            x[l, t, c] = np.float16((int(next(d)) - 32) * step)


def test_open_words_and_carries_match_the_oracle():
    """Symbol strings whose coding interval keeps straddling a byte boundary for
    hundreds of symbols (what the decoder reads from a prefix followed by zero
    bytes), planted into chosen channels: the encoder holds long runs of
    all-ones words open and settles them by a carry or not (the flush, or
    random symbols after the run).  GPU blobs equal the oracle's."""
    w = gu.workload(layers=1, tokens=2000, channels=64, chunk_tokens=2000, group_tokens=10,
                    layer_group_end=(1,), layer_step=(0.5,), qualities=(0,), seed=21)
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    tv = oracle.tables_view(ot)
    n = w.tokens - (w.tokens + w.group_tokens - 1) // w.group_tokens
    rng = np.random.default_rng(5)
    k2, v2 = k.copy(), v.copy()
    planted = {}
    for c in range(0, 64, 3):
        kv = c % 2
        freq = tv.freq[0][kv, 0, c]
        pre = rng.integers(0, 256, int(rng.integers(1, 10)), dtype=np.uint8).tobytes()
        head = int(rng.integers(n // 2, n + 1))
        s1 = oracle.rc_decode(pre + b"\0" * 4000, head, freq)[0].astype(np.int64)
        s2 = rng.choice(64, n - head, p=freq / freq.sum())
        syms = np.concatenate([s1, s2])
        plant_symbols(k2 if kv == 0 else v2, tv, kv, 0, c, 0, syms, w.group_tokens)
        planted[(kv, c)] = syms
    _, got = oracle.chunk_symbols(ot, k2, v2, 0, 0)
    for (kv, c), syms in planted.items():
        col = got[kv, 0, :, c]
        assert np.array_equal(col[col != 255], syms), ("planting failed", kv, c)
    ob = oracle.encode_chunk(ot, k2, v2, 0, 0)
    # the planted streams do hold long runs of all-ones or all-zeros words
    bv = oracle.blob_view(ob)
    runs = 0
    for (kv, c) in planted:
        words = np.frombuffer(oracle.stream_bytes(bv, kv, 0, c, extra_words=0), ">u4")
        same = (words == 0xFFFFFFFF) | (words == 0)
        runs += int(np.convolve(same, np.ones(4, int), "valid").max(initial=0) >= 4)
    assert runs >= len(planted) // 2, runs
    import kv_cache_compression_anchor_amd as cg
    out = gu.torch().empty(cg.cg_encode_bound(tab, 0), dtype=gu.torch().uint8, device="cuda")
    nb = cg.cg_encode(tab, gu.to_dev(k2), gu.to_dev(v2), 0, 0, out)
    gb = out[:nb].cpu().numpy().tobytes()
    assert gb == ob, gu.first_difference(gb, ob)
    kg, vg, st = gu.gpu_decode(tab, [out[:nb]], k.shape)
    ko, vo, bad = gu.oracle_decode(ot, [ob], k.shape)
    assert st == 0 and not bad and gu.same_bits(kg, ko) and gu.same_bits(vg, vo)


def test_symbols_outside_the_search_window():
    """The decoder bisects the 16 symbols [24, 40) around the zero delta first
    and lets a wave redo a symbol with the full search when some lane's symbol
    lies outside.  Planted delta strings: one lane of a wave with only tail
    symbols (the rest of the wave inside the window), the window's edges and the
    alphabet's ends in turn (23, 24, 39, 40, 0, 63), and symbols on the inner
    edges only.  Blobs and the decode through both kernels (two chunks of a
    quality in one workgroup, and one chunk per workgroup) equal the oracle's."""
    w = gu.workload(layers=1, tokens=2000, channels=128, chunk_tokens=1000, group_tokens=10,
                    layer_group_end=(1,), layer_step=(0.5,), qualities=(0,), seed=23)
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    tv = oracle.tables_view(ot)
    n = w.tokens - w.tokens // w.group_tokens
    rng = np.random.default_rng(9)
    tails = np.concatenate([np.arange(0, 24), np.arange(40, 64)])
    edges = np.resize(np.array([23, 24, 39, 40, 0, 63, 32, 31]), n)
    inner = np.resize(np.array([24, 39]), n)
    plan = {(0, 5): rng.choice(tails, n), (0, 70): edges, (1, 3): inner, (1, 127): rng.choice(tails, n)}
    k2, v2 = k.copy(), v.copy()
    for (kv, c), syms in plan.items():
        plant_symbols(k2 if kv == 0 else v2, tv, kv, 0, c, 0, syms, w.group_tokens)
    for ch in range(w.n_chunks):
        _, got = oracle.chunk_symbols(ot, k2, v2, ch, 0)
        for (kv, c), syms in plan.items():
            col = got[kv, 0, :, c]
            assert np.array_equal(col[col != 255], syms[ch * 900:(ch + 1) * 900]), ("planting failed", kv, c)
    kd2, vd2 = gu.to_dev(k2), gu.to_dev(v2)
    dblobs, obs = [], []
    for ch in range(w.n_chunks):
        dblob, gb = gu.gpu_encode(tab, kd2, vd2, ch, 0)
        ob = oracle.encode_chunk(ot, k2, v2, ch, 0)
        assert gb == ob, ("blob differs", ch, gu.first_difference(gb, ob))
        dblobs.append(dblob)
        obs.append(ob)
    ko, vo, bad = gu.oracle_decode(ot, obs, k.shape)
    assert not bad
    kg, vg, st = gu.gpu_decode(tab, dblobs, k.shape)  # both chunks in one workgroup
    assert st == 0 and gu.same_bits(kg, ko) and gu.same_bits(vg, vo)
    for ch in range(w.n_chunks):  # one chunk per workgroup
        kg, vg, st = gu.gpu_decode(tab, [dblobs[ch]], k.shape)
        rk, rv, _ = gu.oracle_decode(ot, [obs[ch]], k.shape)
        assert st == 0 and gu.same_bits(kg, rk) and gu.same_bits(vg, rv), ch


def test_default_layer_groups_match_the_explicit_split():
    """n_layer_groups = 0 (the binding's layer_group_end=None): the library's
    default split of 48 layers is 15 / 30 / 48, the tables equal the oracle's
    with those ends written out, and cg_tables_params reports them."""
    import kv_cache_compression_anchor_amd as cg
    w = gu.workload(layers=48, tokens=200, channels=64, chunk_tokens=200,
                    layer_group_end=(15, 30, 48), qualities=(0,))
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    p = cg.make_params(w.layers, w.tokens, w.channels, w.chunk_tokens, w.group_tokens, None,
                       w.layer_step, w.quality_mult, w.quality_mask)
    tab = cg.cg_build_tables(p, kd, vd)
    assert cg.cg_tables_serialize(tab) == oracle.build_tables(oracle.params_for(w), k, v)
    got = cg.cg_tables_params(tab)
    assert got.n_layer_groups == 3 and list(got.layer_group_end) == [15, 30, 48]
