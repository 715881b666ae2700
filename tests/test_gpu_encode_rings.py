"""GPU parity on geometries that drive the encoder's launch choices: a wide,
single-chunk row set whose workgroups (one wave each, sixteen per compute unit)
take the 4-word output rings; the same with three qualities in one batch
(several groups of one wave per launch); and a deep, many-chunk set whose
batch the planner cuts from 5 to 4 blobs per launch so that 8-word rings fit.
Every blob of the batch and the decode of a selection must equal the
oracle's byte for byte, with raw and with coded anchors."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = {
    # 2 x 32 x 64 = 4096 one-wave workgroups per blob
    "wide_one_chunk": dict(L=32, T=64, C=4096, chunk=64, G=10, ends=(10, 20, 32),
                           steps=(0.5, 1.0, 1.5), qualities=(0,)),
    "wide_three_qualities": dict(L=32, T=64, C=4096, chunk=64, G=10, ends=(10, 20, 32),
                                 steps=(0.5, 1.0, 1.5), qualities=(0, 1, 2)),
    # 2 x 48 x 16 = 1536 waves per blob: 5 blobs fit the device at once, 4 fit its LDS
    "deep_six_chunks": dict(L=48, T=96, C=1024, chunk=16, G=8, ends=(16, 32, 48),
                            steps=(0.5, 1.0, 1.5), qualities=(1,)),
}


def workload(name):
    c = CASES[name]
    return synth.Workload(name, c["L"], c["T"], c["C"], seed=7, rho=0.85, outlier_frac=0.02,
                          chunk_tokens=c["chunk"], group_tokens=c["G"], layer_group_end=c["ends"],
                          layer_step=c["steps"], qualities=c["qualities"])


@pytest.mark.parametrize("coding", [0, 1])
@pytest.mark.parametrize("name", sorted(CASES))
def test_encode_launch_shapes(name, coding):
    import kv_cache_compression_anchor_amd as cg
    w = workload(name)
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd, anchor_coding=coding)
    ot = oracle.build_tables(oracle.params_for(w, anchor_coding=coding), k, v)
    assert cg.cg_tables_serialize(tab) == ot
    jobs = [(c, q) for c in range(w.n_chunks) for q in w.qualities]
    t = gu.torch()
    outs = [t.empty(cg.cg_encode_bound(tab, c), dtype=t.uint8, device="cuda") for c, _ in jobs]
    lens = cg.cg_encode_batch(tab, kd, vd, [c for c, _ in jobs], [q for _, q in jobs], outs)
    blobs = {}
    for (c, q), o, n in zip(jobs, outs, lens):
        got = o[:n].cpu().numpy().tobytes()
        want = oracle.encode_chunk(ot, k, v, c, q)
        assert got == want, (name, coding, c, q, gu.first_difference(got, want))
        blobs[(c, q)] = (o[:n], want)
    sel = [(c, w.qualities[c % len(w.qualities)]) for c in range(w.n_chunks)]
    kg, vg, st = gu.gpu_decode(tab, [blobs[j][0] for j in sel], k.shape)
    ko, vo, bad = gu.oracle_decode(ot, [blobs[j][1] for j in sel], k.shape)
    assert st == 0 and not bad
    assert gu.same_bits(kg, ko) and gu.same_bits(vg, vo), (name, coding)
