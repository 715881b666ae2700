"""The library's per-device state: the encode workspace (stream scratch,
lengths, status words) that every cg_encode_batch on a device shares, and the
stream-ordered memory pool that holds each tables handle's device copies and the
coded-anchor decode workspace.  Batches of two tables handles of different
shapes run from two host threads at once (they take turns on the workspace,
which grows to the larger one) and give the oracle's blobs; tables freed and
built again in a loop keep giving the oracle's bytes (the pool hands freed
blocks back)."""
import threading

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _setup(w):
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    jobs = [(c, q) for c in range(w.n_chunks) for q in w.qualities]
    want = [oracle.encode_chunk(ot, k, v, c, q) for c, q in jobs]
    return kd, vd, tab, ot, jobs, want


def _batch(tab, kd, vd, jobs, stream=None):
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    outs = [t.empty(cg.cg_encode_bound(tab, c), dtype=t.uint8, device="cuda") for c, _ in jobs]
    lens = cg.cg_encode_batch(tab, kd, vd, [c for c, _ in jobs], [q for _, q in jobs], outs,
                              stream)
    if stream is not None:
        stream.synchronize()
    return [o[:n].cpu().numpy().tobytes() for o, n in zip(outs, lens)]


def test_concurrent_batches_on_two_handles():
    a = _setup(gu.workload(tokens=1000, channels=100, chunk_tokens=384))
    b = _setup(gu.workload(tokens=700, channels=200, chunk_tokens=256, layers=2,
                           layer_group_end=(1, 2), layer_step=(0.5, 1.5), seed=11))
    t = gu.torch()
    results, errors = {}, []

    def run(name, s):
        kd, vd, tab, _, jobs, _ = s
        stream = t.cuda.Stream()
        try:
            for rep in range(3):
                results[(name, rep)] = _batch(tab, kd, vd, jobs, stream)
        except Exception as e:  # reported below
            errors.append(repr(e))

    th = [threading.Thread(target=run, args=(n, s)) for n, s in (("a", a), ("b", b))]
    for x in th:
        x.start()
    for x in th:
        x.join()
    assert not errors, errors
    for name, s in (("a", a), ("b", b)):
        want = s[5]
        for rep in range(3):
            got = results[(name, rep)]
            for i, (g, o) in enumerate(zip(got, want)):
                assert g == o, (name, rep, s[4][i], gu.first_difference(g, o))


def test_tables_built_and_freed_in_a_loop():
    import kv_cache_compression_anchor_amd as cg
    ws = [gu.workload(tokens=600, channels=70, chunk_tokens=200),
          gu.workload(tokens=1200, channels=160, chunk_tokens=512, seed=5)]
    data = []
    for w in ws:
        k, v = synth.gen_kv(w)
        data.append((w, gu.to_dev(k), gu.to_dev(v),
                     oracle.build_tables(oracle.params_for(w), k, v)))
    for rep in range(6):
        w, kd, vd, ot = data[rep % 2]
        for coding in (0, 1):
            tab = gu.gpu_tables(w, kd, vd, anchor_coding=coding)
            got = cg.cg_tables_serialize(tab)
            if coding == 0:
                assert got == ot, (rep, gu.first_difference(got, ot))
            else:
                ot1 = oracle.build_tables(oracle.params_for(w, anchor_coding=1),
                                          kd.cpu().numpy(), vd.cpu().numpy())
                assert got == ot1, (rep, gu.first_difference(got, ot1))
            cg.cg_tables_free(tab)


def test_release_cached_then_work_again():
    """cg_release_cached frees the workspaces and trims the pool; the next
    build, encode and coded-anchor decode allocate again and still give the
    oracle's bytes."""
    import kv_cache_compression_anchor_amd as cg
    w = gu.workload(tokens=900, channels=130, chunk_tokens=300)
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    ot = oracle.build_tables(oracle.params_for(w, anchor_coding=1), k, v)
    jobs = [(c, q) for c in range(w.n_chunks) for q in w.qualities]
    want = [oracle.encode_chunk(ot, k, v, c, q) for c, q in jobs]
    for rep in range(3):
        tab = gu.gpu_tables(w, kd, vd, anchor_coding=1)
        assert cg.cg_tables_serialize(tab) == ot
        got = _batch(tab, kd, vd, jobs)
        assert got == want, rep
        # one blob per chunk (qualities in turn), so no two write the same rows
        sel = [jobs.index((c, w.qualities[c % len(w.qualities)])) for c in range(w.n_chunks)]
        dev = [gu.to_dev(np.frombuffer(got[i], dtype=np.uint8).copy()) for i in sel]
        kg, vg, st = gu.gpu_decode(tab, dev, k.shape)
        ko, vo, bad = gu.oracle_decode(ot, [want[i] for i in sel], k.shape)
        assert st == 0 and not bad
        assert gu.same_bits(kg, ko) and gu.same_bits(vg, vo)
        cg.cg_release_cached()
        cg.cg_tables_free(tab)
