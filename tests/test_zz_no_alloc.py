"""cg_encode_batch_noalloc (static device scratch, no allocation) against
cg_encode_batch on the same inputs: every blob byte and length identical, on
two calls in a row, the second with a smaller input; a shape whose rows take
several ranges of the static scratch; and a chunk whose single row exceeds the
static scratch, rejected before any launch."""
import numpy as np
import pytest

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def both_ways(w, jobs):
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    chunks = [c for c, _ in jobs]
    quals = [q for _, q in jobs]
    outs_a = [t.full((cg.cg_encode_bound(tab, c),), 0xA5, dtype=t.uint8, device="cuda")
              for c in chunks]
    outs_b = [t.full((cg.cg_encode_bound(tab, c),), 0x5A, dtype=t.uint8, device="cuda")
              for c in chunks]
    la = cg.cg_encode_batch(tab, kd, vd, chunks, quals, outs_a)
    lb = cg.cg_encode_batch_noalloc(tab, kd, vd, chunks, quals, outs_b)
    assert la == lb
    for (c, q), oa, ob, n in zip(jobs, outs_a, outs_b, la):
        assert n > 64
        a = oa[:n].cpu().numpy()
        b = ob[:n].cpu().numpy()
        assert np.array_equal(a, b), ("blob differs", c, q, int(np.argmax(a != b)))


def test_two_calls_in_a_row_the_second_smaller():
    w1 = gu.workload()  # 3 layers, 1000 tokens (3 chunks, the last ragged), 100 channels
    both_ways(w1, [(c, q) for c in range(w1.n_chunks) for q in w1.qualities])
    w2 = gu.workload(layers=2, tokens=300, channels=64, chunk_tokens=128,
                     layer_group_end=(1, 2), layer_step=(0.5, 1.5), qualities=(0, 2))
    both_ways(w2, [(c, q) for c in range(w2.n_chunks) for q in w2.qualities])


def test_rows_in_several_ranges_of_the_static_scratch():
    # 4096 channels x 1536 tokens: a (kv, layer) row takes about 10.7 MB of
    # stream scratch, so the 32 rows of this blob go through the static
    # scratch in two ranges
    w = synth.workload("llama7b", layers=16, layer_group_end=(5, 10, 16), qualities=(0, 2))
    both_ways(w, [(0, 0), (0, 2)])


def test_a_row_beyond_the_static_scratch_is_rejected():
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    L, T, C = 1, 8192, 65536
    g = t.Generator(device="cuda").manual_seed(3)
    kd = t.randn((L, T, C), generator=g, device="cuda").to(t.float16)
    vd = t.randn((L, T, C), generator=g, device="cuda").to(t.float16)
    p = cg.make_params(L, T, C, 8192, 10, (1,), (0.5,))
    tab = cg.cg_build_tables(p, kd, vd)
    out = t.zeros(cg.cg_encode_bound(tab, 0), dtype=t.uint8, device="cuda")
    with pytest.raises(cg.CgError) as e:
        cg.cg_encode_batch_noalloc(tab, kd, vd, [0], [0], [out])
    assert e.value.code == cg.CG_E_CAPACITY and "static scratch" in str(e.value)
    assert int(out.count_nonzero()) == 0  # nothing was launched
