"""GPU parity on seeded random geometries: layers, tokens, channels, chunk and
group sizes, layer groups, the qualities built and both anchor formats are
drawn from a fixed seed per case.  Tables, every blob of one cg_encode_batch
call and the decode of a selection (one quality per chunk, the qualities in
turn) must equal the oracle's byte for byte."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def random_workload(seed):
    r = np.random.default_rng(1000 + seed)
    L = int(r.integers(1, 5))
    T = int(r.integers(1, 700))
    C = int(r.integers(1, 200))
    chunk = int(r.integers(1, T + 1))
    G = int(r.integers(1, min(12, chunk) + 1))  # the parameters require G <= chunk_tokens
    ng = int(r.integers(1, min(L, 3) + 1))
    ends = sorted(r.choice(np.arange(1, L), size=ng - 1, replace=False).tolist()) if ng > 1 else []
    ends = tuple(int(e) for e in ends) + (L,)
    steps = tuple(float(x) for x in np.round(r.uniform(0.3, 2.0, size=ng), 2))
    qs = tuple(sorted(r.choice(3, size=int(r.integers(1, 4)), replace=False).tolist()))
    w = synth.Workload("random", L, T, C, seed=int(seed), rho=float(r.uniform(0.5, 0.95)),
                       outlier_frac=float(r.choice([0.0, 0.03])), chunk_tokens=chunk,
                       group_tokens=G, layer_group_end=ends, layer_step=steps,
                       qualities=tuple(int(q) for q in qs))
    return w, int(r.integers(0, 2))


@pytest.mark.parametrize("seed", range(40))
def test_random_geometry(seed):
    import kv_cache_compression_anchor_amd as cg
    w, coding = random_workload(seed)
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd, anchor_coding=coding)
    ot = oracle.build_tables(oracle.params_for(w, anchor_coding=coding), k, v)
    gt = cg.cg_tables_serialize(tab)
    assert gt == ot, (w, coding, gu.first_difference(gt, ot))
    jobs = [(c, q) for c in range(w.n_chunks) for q in w.qualities]
    t = gu.torch()
    outs = [t.empty(cg.cg_encode_bound(tab, c), dtype=t.uint8, device="cuda") for c, _ in jobs]
    lens = cg.cg_encode_batch(tab, kd, vd, [c for c, _ in jobs], [q for _, q in jobs], outs)
    blobs = {}
    for (c, q), o, n in zip(jobs, outs, lens):
        got = o[:n].cpu().numpy().tobytes()
        want = oracle.encode_chunk(ot, k, v, c, q)
        assert got == want, (w, coding, c, q, gu.first_difference(got, want))
        blobs[(c, q)] = (o[:n], want)
    sel = [(c, w.qualities[c % len(w.qualities)]) for c in range(w.n_chunks)]
    kg, vg, st = gu.gpu_decode(tab, [blobs[j][0] for j in sel], k.shape)
    ko, vo, bad = gu.oracle_decode(ot, [blobs[j][1] for j in sel], k.shape)
    assert st == 0 and not bad
    assert gu.same_bits(kg, ko) and gu.same_bits(vg, vo), (w, coding)
