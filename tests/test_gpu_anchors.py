"""GPU parity of coded anchors (tables version 2, blobs version 3) with the
oracle: the anchor tables, every blob byte and every decoded fp16 bit; both
decoder kernels and the paged and streamed decodes reading anchors that
k_anchor_decode wrote; the allocation-free encoder; the argument and format
checks; corrupt anchor streams flagged without fault; and a full-size chunk of
the Mistral-7B-shape workload."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def coded_setup(w):
    import kv_cache_compression_anchor_amd as cg
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd, anchor_coding=1)
    ot = oracle.build_tables(oracle.params_for(w, anchor_coding=1), k, v)
    gt = cg.cg_tables_serialize(tab)
    assert gt == ot, ("tables differ", gu.first_difference(gt, ot))
    assert tab.id == oracle.tables_id(ot)
    return k, v, kd, vd, tab, ot


def run_all(w):
    k, v, kd, vd, tab, ot = coded_setup(w)
    for ch in range(w.n_chunks):
        for q in w.qualities:
            dblob, gb = gu.gpu_encode(tab, kd, vd, ch, q)
            ob = oracle.encode_chunk(ot, k, v, ch, q)
            assert oracle.parse_blob_header(ob)["version"] == 3
            assert gb == ob, ("blob differs", ch, q, gu.first_difference(gb, ob))
            kg, vg, st = gu.gpu_decode(tab, [dblob], k.shape)
            ko, vo, bad = gu.oracle_decode(ot, [ob], k.shape)
            assert st == 0 and not bad
            assert gu.same_bits(kg, ko) and gu.same_bits(vg, vo), ("decode differs", ch, q)
    return k, v, kd, vd, tab, ot


def test_tiny_workload():
    run_all(synth.workload("tiny"))


def test_multi_chunk_ragged_three_qualities():
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


@pytest.mark.parametrize("group_tokens", [10, 7])
def test_selection_decoded_in_one_call(group_tokens):
    """Chunks of mixed qualities in one cg_decode_async call: pairs of one
    quality take the LDS-window kernel, a lone chunk the register-buffer
    kernel; all read anchors from the decoded anchor streams."""
    w = gu.workload(tokens=2000, chunk_tokens=256, channels=192, group_tokens=group_tokens)
    k, v, kd, vd, tab, ot = coded_setup(w)
    sel = [(ch, [0, 0, 1, 1, 2, 0, 1, 2][ch]) for ch in range(w.n_chunks)]
    dev, ref = [], []
    for ch, q in sel:
        db, gb = gu.gpu_encode(tab, kd, vd, ch, q)
        ob = oracle.encode_chunk(ot, k, v, ch, q)
        assert gb == ob
        dev.append(db)
        ref.append(ob)
    kg, vg, st = gu.gpu_decode(tab, dev, k.shape)
    ko, vo, bad = gu.oracle_decode(ot, ref, k.shape)
    assert st == 0 and not bad
    assert gu.same_bits(kg, ko) and gu.same_bits(vg, vo)


def test_encode_batch_and_noalloc_match_the_oracle():
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    w = gu.workload(tokens=900, chunk_tokens=300, channels=150)
    k, v, kd, vd, tab, ot = coded_setup(w)
    jobs = [(ch, q) for ch in range(w.n_chunks) for q in w.qualities]
    outs = [t.empty(cg.cg_encode_bound(tab, ch), dtype=t.uint8, device="cuda") for ch, _ in jobs]
    lens = cg.cg_encode_batch(tab, kd, vd, [j[0] for j in jobs], [j[1] for j in jobs], outs)
    outs2 = [t.empty_like(o) for o in outs]
    lens2 = cg.cg_encode_batch_noalloc(tab, kd, vd, [j[0] for j in jobs], [j[1] for j in jobs],
                                       outs2)
    for (ch, q), o, n, o2, n2 in zip(jobs, outs, lens, outs2, lens2):
        ob = oracle.encode_chunk(ot, k, v, ch, q)
        assert o[:n].cpu().numpy().tobytes() == ob
        assert n2 == n and o2[:n2].cpu().numpy().tobytes() == ob


def test_paged_and_streamed_decodes():
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    w = gu.workload(tokens=1000, chunk_tokens=256, channels=128, seed=31)
    k, v, kd, vd, tab, ot = coded_setup(w)
    sel = [(ch, ch % 3) for ch in range(w.n_chunks)]
    dev = [gu.gpu_encode(tab, kd, vd, ch, q)[0] for ch, q in sel]
    ref = [oracle.encode_chunk(ot, k, v, ch, q) for ch, q in sel]
    # paged: pages of 16 tokens, in reverse order
    P = 16
    n_pages = -(-w.tokens // P)
    table = np.arange(n_pages, dtype=np.int32)[::-1].copy()
    L, T, Cc = k.shape
    kp = t.zeros((L, n_pages, P, Cc), dtype=t.float16, device="cuda")
    vp = t.zeros_like(kp)
    st = t.zeros(1, dtype=t.int32, device="cuda")
    infos = [cg.cg_chunk_info_parse(b[:64].cpu()) for b in dev]
    assert all(i.version == 3 for i in infos)
    cg.cg_decode_paged_async(tab, dev, infos, kp, vp, P, gu.to_dev(table), st)
    t.cuda.synchronize()
    rk = np.zeros((L, n_pages, P, Cc), np.float16)
    rv = np.zeros_like(rk)
    for b in ref:
        c, bad = oracle.decode_blob_paged(ot, b, rk, rv, P, table)
        assert not c and not bad
    assert int(st.item()) == 0
    assert gu.same_bits(kp.cpu().numpy(), rk) and gu.same_bits(vp.cpu().numpy(), rv)
    # streamed from pinned host memory through two staging slots
    host = [b.cpu().pin_memory() for b in dev]
    slot = max((b.numel() + 255) // 256 * 256 for b in dev)
    ko, vo = t.zeros_like(kd), t.zeros_like(vd)
    st.zero_()
    stage = t.empty(2 * slot, dtype=t.uint8, device="cuda")
    cs, ks = t.cuda.Stream(), t.cuda.Stream()
    cg.cg_decode_streamed(tab, host, infos, ko, vo, stage, st, cs, ks)
    ks.synchronize()
    rk2, rv2, bad = gu.oracle_decode(ot, ref, k.shape)
    assert int(st.item()) == 0 and not bad
    assert gu.same_bits(ko.cpu().numpy(), rk2) and gu.same_bits(vo.cpu().numpy(), rv2)


def test_formats_and_tables_must_agree():
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    w = gu.workload(layers=1, tokens=200, channels=64, chunk_tokens=100, layer_group_end=(1,),
                    layer_step=(0.5,), qualities=(0,))
    k, v, kd, vd, tab, ot = coded_setup(w)
    raw = gu.gpu_tables(w, kd, vd)
    coded_blob, _ = gu.gpu_encode(tab, kd, vd, 0, 0)
    raw_blob, _ = gu.gpu_encode(raw, kd, vd, 0, 0)
    ko, vo = t.zeros_like(kd), t.zeros_like(vd)
    st = t.zeros(1, dtype=t.int32, device="cuda")
    for tb, b in ((raw, coded_blob), (tab, raw_blob)):
        info = cg.cg_chunk_info_parse(b[:64].cpu())
        with pytest.raises(cg.CgError) as e:
            cg.cg_decode_async(tb, [b], [info], ko, vo, st)
        assert e.value.code == cg.CG_E_MISMATCH
    # serialised coded tables come back with their anchor tables and id
    tab2 = cg.cg_tables_deserialize(cg.cg_tables_serialize(tab))
    assert tab2.id == tab.id and cg.cg_tables_params(tab2).anchor_coding == 1
    kg, vg, s2 = gu.gpu_decode(tab2, [coded_blob], k.shape)
    ko2, vo2, _ = gu.oracle_decode(ot, [oracle.encode_chunk(ot, k, v, 0, 0)], k.shape)
    assert s2 == 0 and gu.same_bits(kg, ko2) and gu.same_bits(vg, vo2)


def test_corrupt_anchor_streams_are_flagged_without_fault():
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    w = gu.workload(layers=2, tokens=300, channels=128, chunk_tokens=300,
                    layer_group_end=(1, 2), layer_step=(0.5, 1.0), qualities=(0,))
    k, v, kd, vd, tab, ot = coded_setup(w)
    blob, hb = gu.gpu_encode(tab, kd, vd, 0, 0)
    bv = oracle.blob_view(hb)
    L, Cc = w.layers, w.channels
    off_len = 64 + 16 * L  # lengths of the 4L rows after the row offsets
    flagged = 0
    rng = np.random.default_rng(3)
    for trial in range(6):
        bad = blob.clone()
        if trial % 2:
            # an anchor stream's length far past the payload
            at = off_len + 2 * (2 * L * Cc + 5)
            bad[at: at + 2] = t.tensor([0xFF, 0xFF], dtype=t.uint8)
        else:
            start = bv.payload_offset + 4 * int(bv.anchor_row_offset[0, 0])
            pos = start + rng.integers(0, 4 * int(bv.anchor_lengths.astype(np.int64).sum()), 64)
            bad[t.as_tensor(pos, device="cuda")] ^= 0x5A
        ko, vo = t.zeros_like(kd), t.zeros_like(vd)
        st = t.zeros(1, dtype=t.int32, device="cuda")
        info = cg.cg_chunk_info_parse(bad[:64].cpu())
        cg.cg_decode_async(tab, [bad], [info], ko, vo, st)
        t.cuda.synchronize()
        flagged += int(st.item()) != 0
        if trial % 2:
            assert int(st.item()) != 0
    assert flagged >= 3


def test_full_size_chunk_of_the_mistral_workload():
    """One chunk of the Mistral-7B-shape 9K workload at every quality, coded
    anchors: blobs byte-identical with the oracle, the chunk decoded in the
    two-chunk launch the benchmark times, and a bit-identical decode."""
    import kv_cache_compression_anchor_amd as cg
    w = synth.workload("mistral7b_9k")
    k, v, kd, vd, tab, ot = coded_setup(w)
    dev, ref = [], []
    for ch, q in ((0, 0), (1, 0), (2, 1), (5, 2)):
        db, gb = gu.gpu_encode(tab, kd, vd, ch, q)
        ob = oracle.encode_chunk(ot, k, v, ch, q)
        assert gb == ob, ("blob differs", ch, q, gu.first_difference(gb, ob))
        dev.append(db)
        ref.append(ob)
    kg, vg, st = gu.gpu_decode(tab, dev, k.shape)
    ko, vo, bad = gu.oracle_decode(ot, ref, k.shape)
    assert st == 0 and not bad
    assert gu.same_bits(kg, ko) and gu.same_bits(vg, vo)
