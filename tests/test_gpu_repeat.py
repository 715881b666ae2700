"""Decoding is a pure function of the blobs and tables: the same selection
decoded several times in a row, into fresh buffers, gives bitwise the same K and
V every time and never flags a stream; encoding the chunks twice gives the same
blobs.  Run at full size on both decoder kernels: the register-buffer one (one
chunk per workgroup, Llama-7B shape) and the LDS-window one (several chunks of
a quality per workgroup, the Mistral-7B 9K selection).  Parity of the values
themselves with the oracle is the subject of the full-size test; this one
catches a kernel whose result changes from run to run, which a single
comparison can miss."""
import pytest

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

REPEATS = 4


@pytest.mark.parametrize("name", ["llama7b", "mistral7b_9k"])
def test_repeated_decodes_are_identical(name):
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    w = synth.workload(name)
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    sel = w.selection()
    outs = [t.empty(cg.cg_encode_bound(tab, c), dtype=t.uint8, device="cuda") for c in range(len(sel))]
    sizes = cg.cg_encode_batch(tab, kd, vd, list(range(len(sel))), list(sel), outs)
    blobs = [o[:n] for o, n in zip(outs, sizes)]
    again = [t.empty(cg.cg_encode_bound(tab, c), dtype=t.uint8, device="cuda") for c in range(len(sel))]
    sizes2 = cg.cg_encode_batch(tab, kd, vd, list(range(len(sel))), list(sel), again)
    assert list(sizes2) == list(sizes)
    for b, o, n in zip(blobs, again, sizes2):
        assert t.equal(b, o[:n]), (name, "encode differs")
    infos = [cg.cg_chunk_info_parse(b[:64].cpu()) for b in blobs]
    first = None
    for rep in range(REPEATS):
        ko, vo = t.empty_like(kd), t.empty_like(vd)
        st = t.zeros(1, dtype=t.int32, device="cuda")
        cg.cg_decode_async(tab, blobs, infos, ko, vo, st)
        t.cuda.synchronize()
        assert int(st.item()) == 0, (name, rep, "a stream was flagged")
        kb, vb = ko.view(t.int16), vo.view(t.int16)
        if first is None:
            first = (kb, vb)
        else:
            assert t.equal(kb, first[0]) and t.equal(vb, first[1]), (name, rep, "decode differs")
