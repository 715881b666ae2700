"""GPU parity of the pooled table groupings (cg_build_tables_grouped): the
tables, every blob coded with them and the decoded values equal the oracle's,
for every grouping, on a shape spanning several 64-channel blocks, layers of
all three groups, and a ragged last chunk."""
import pytest

import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("grouping", [0, 1, 2, 3])
def test_grouped_tables_blobs_and_decode_match_the_oracle(grouping):
    import kv_cache_compression_anchor_amd as cg
    w = gu.workload(layers=5, channels=130, layer_group_end=(1, 3, 5))
    k, v = gu.synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = cg.cg_build_tables_grouped(gu.params_of(w), grouping, kd, vd)
    ot = oracle.build_tables_grouped(oracle.params_for(w), k, v, grouping, threads=8)
    gt = cg.cg_tables_serialize(tab)
    assert gt == ot, ("tables differ", gu.first_difference(gt, ot))
    for q in w.qualities:
        blobs, obs = [], []
        for ch in range(w.n_chunks):
            b, gb = gu.gpu_encode(tab, kd, vd, ch, q)
            ob = oracle.encode_chunk(ot, k, v, ch, q)
            assert gb == ob, ("blob differs", grouping, ch, q, gu.first_difference(gb, ob))
            blobs.append(b)
            obs.append(ob)
        ko, vo, st = gu.gpu_decode(tab, blobs, k.shape)
        rk, rv, bad = gu.oracle_decode(ot, obs, k.shape)
        assert st == 0 and not bad
        assert gu.same_bits(ko, rk) and gu.same_bits(vo, rv)


def test_unknown_grouping_is_rejected():
    import kv_cache_compression_anchor_amd as cg
    w = gu.workload(layers=1, tokens=20, channels=8)
    k, v = gu.synth.gen_kv(w)
    with pytest.raises(cg.CgError) as e:
        cg.cg_build_tables_grouped(gu.params_of(w), 4, gu.to_dev(k), gu.to_dev(v))
    assert e.value.code == cg.CG_E_INVAL
