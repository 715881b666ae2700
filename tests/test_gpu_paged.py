"""GPU parity of the decode into paged K/V pools (cg_decode_paged_async) with
the oracle's decode_blob_paged: every pool byte equal, on both decoder kernels
(one chunk per call takes the register-buffer kernel, several chunks of a
quality the LDS-window kernel), the unrolled and the runtime group sizes, page
sizes from one token to more than the context, ragged channel blocks, spare
pages that must stay untouched, block-table entries outside the pool (flagged,
skipped), the argument checks, and the two full-size selections in the launch
configuration the benchmark times."""
import ctypes as C

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

FILL = 0x7E5A  # a NaN pattern the codec never writes


def fill_pools(shape):
    k = np.full(shape, FILL, np.uint16).view(np.float16)
    v = np.full(shape, FILL, np.uint16).view(np.float16)
    return k, v


def coded(w, qs):
    """GPU and oracle tables and blobs of chunks 0.. at qualities qs."""
    import kv_cache_compression_anchor_amd as cg
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    assert cg.cg_tables_serialize(tab) == ot
    dblobs, oblobs = [], []
    for ch, q in enumerate(qs):
        db, gb = gu.gpu_encode(tab, kd, vd, ch, q)
        ob = oracle.encode_chunk(ot, k, v, ch, q)
        assert gb == ob, ("blob differs", ch, q)
        dblobs.append(db)
        oblobs.append(ob)
    return k.shape, tab, ot, dblobs, oblobs


def gpu_paged(tab, dblobs, calls, pool_shape, P, table):
    """Decode the blobs into FILL-initialised pools, calls = lists of blob indices
    per cg_decode_paged_async call; returns (k, v, status)."""
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    kf, vf = fill_pools(pool_shape)
    kp, vp = gu.to_dev(kf), gu.to_dev(vf)
    tb = gu.to_dev(np.asarray(table, np.int32))
    st = t.zeros(1, dtype=t.int32, device="cuda")
    infos = [cg.cg_chunk_info_parse(b[:64].cpu()) for b in dblobs]
    for idx in calls:
        cg.cg_decode_paged_async(tab, [dblobs[i] for i in idx], [infos[i] for i in idx], kp, vp, P,
                                 tb, st)
    t.cuda.synchronize()
    return kp.cpu().numpy(), vp.cpu().numpy(), int(st.item())


def oracle_paged(ot, oblobs, pool_shape, P, table):
    k, v = fill_pools(pool_shape)
    corrupt = bad = False
    for b in oblobs:
        c, p = oracle.decode_blob_paged(ot, b, k, v, P, np.asarray(table, np.int32))
        corrupt |= c
        bad |= p
    return k, v, corrupt, bad


def check(shape, tab, ot, dblobs, oblobs, calls, P, table, n_pages, want_status=0):
    L, T, Cc = shape
    ps = (L, n_pages, P, Cc)
    kg, vg, st = gpu_paged(tab, dblobs, calls, ps, P, table)
    ko, vo, corrupt, bad = oracle_paged(ot, oblobs, ps, P, table)
    assert not corrupt
    assert st == want_status and bad == bool(want_status & 2)
    assert gu.same_bits(kg, ko) and gu.same_bits(vg, vo), "pools differ"


def perm_table(T, P, spare, seed):
    nb = -(-T // P)
    return np.random.default_rng(seed).permutation(nb + spare)[:nb].astype(np.int32), nb + spare


@pytest.mark.parametrize("G,Cc", [(10, 138), (1, 65), (7, 135), (13, 128), (64, 192)])
@pytest.mark.parametrize("P", [1, 16, 64])
def test_paged_matches_oracle(G, Cc, P):
    w = gu.workload(tokens=1000, chunk_tokens=384, group_tokens=G, channels=Cc)
    shape, tab, ot, dblobs, oblobs = coded(w, [0, 0, 0])
    table, n_pages = perm_table(shape[1], P, spare=5, seed=G * 1000 + P)
    # one chunk per call: register-buffer kernel; all three in one call: window kernel
    check(shape, tab, ot, dblobs, oblobs, [[0], [1], [2]], P, table, n_pages)
    check(shape, tab, ot, dblobs, oblobs, [[0, 1, 2]], P, table, n_pages)


def test_mixed_qualities_and_one_large_page():
    w = gu.workload(tokens=2000, chunk_tokens=256, channels=192)
    qs = [0, 1, 2, 0, 1, 2, 0, 1]
    shape, tab, ot, dblobs, oblobs = coded(w, qs)
    check(shape, tab, ot, dblobs, oblobs, [list(range(8))], 2048, [1], 2)
    table, n_pages = perm_table(shape[1], 8, spare=3, seed=3)
    check(shape, tab, ot, dblobs, oblobs, [list(range(8))], 8, table, n_pages)


def test_entries_outside_the_pool_are_flagged_and_skipped():
    w = gu.workload(tokens=1000, chunk_tokens=384, channels=128)
    shape, tab, ot, dblobs, oblobs = coded(w, [0, 0, 1])
    P = 16
    table, n_pages = perm_table(shape[1], P, spare=2, seed=11)
    table[3] = n_pages          # one past the pool
    table[40] = -1
    table[62] = 1 << 30
    check(shape, tab, ot, dblobs, oblobs, [[0, 1, 2]], P, table, n_pages, want_status=2)
    check(shape, tab, ot, dblobs, oblobs, [[0], [1], [2]], P, table, n_pages, want_status=2)


def test_argument_checks():
    """Checks that need no blob run with zero blobs, so nothing can launch
    whatever they return; the calls with blobs pass pools as large as they
    claim and tables whose entries name page 0, so even a wrongly accepted call
    writes inside the pools."""
    import kv_cache_compression_anchor_amd as cg
    t = gu.torch()
    w = gu.workload(tokens=200, chunk_tokens=100, channels=128)
    shape, tab, ot, dblobs, oblobs = coded(w, [0, 0])
    infos = [cg.cg_chunk_info_parse(b[:64].cpu()) for b in dblobs]
    st = t.zeros(1, dtype=t.int32, device="cuda")
    kp = t.zeros((shape[0], 100, 16, shape[2]), dtype=t.float16, device="cuda")
    vp = t.zeros_like(kp)
    tb = t.zeros(100, dtype=t.int32, device="cuda")

    def call(P, n_pages, n_blocks, nb=0):
        arr = (C.c_void_p * 2)(*[b.data_ptr() for b in dblobs])
        iarr = (cg.cg_chunk_info * 2)(*infos)
        return cg.lib().cg_decode_paged_async(tab.handle, nb, arr, iarr, kp.data_ptr(),
                                              vp.data_ptr(), n_pages, P, tb.data_ptr(), n_blocks,
                                              st.data_ptr(), None)

    assert call(12, 100, 100) == cg.CG_E_INVAL             # not a power of two
    assert call(0, 100, 100) == cg.CG_E_INVAL
    assert call(1 << 17, 100, 100) == cg.CG_E_INVAL
    assert call(16, 0, 100) == cg.CG_E_INVAL
    assert call(16, 100, 0) == cg.CG_E_INVAL
    assert call(16, 1 << 32, 100) == cg.CG_E_INVAL
    assert call(1024, 1 << 13, 100) == cg.CG_E_INVAL       # a layer's pool of 2 GiB
    assert call(1024, (1 << 13) - 1, 100) == cg.CG_OK      # one page less
    assert call(16, 100, 12, nb=2) == cg.CG_E_INVAL        # 200 tokens need 13 blocks of 16
    assert call(16, 100, 13, nb=2) == cg.CG_OK
    t.cuda.synchronize()
    assert int(st.item()) == 0
    # a last channel block narrower than a group: rejected before any launch
    w2 = gu.workload(tokens=200, chunk_tokens=100, channels=130)
    shape2, tab2, _, dblobs2, _ = coded(w2, [0])
    kp2 = t.zeros((shape2[0], 13, 16, shape2[2]), dtype=t.float16, device="cuda")
    tb2 = t.arange(13, dtype=t.int32, device="cuda")
    with pytest.raises(cg.CgError) as e:
        cg.cg_decode_paged_async(tab2, dblobs2, [cg.cg_chunk_info_parse(dblobs2[0][:64].cpu())],
                                 kp2, kp2.clone(), 16, tb2, st)
    assert e.value.code == cg.CG_E_INVAL


@pytest.mark.parametrize("name", ["mistral7b_9k", "llama7b"])
def test_full_size_selection_into_pages(name):
    """The benchmark's selection (Mistral-7B shape: six chunks H, M, L, H, M, L in
    one call, the window kernel; Llama-7B shape: one chunk, the register-buffer
    kernel) into 16-token pages of a shuffled block table with spare pages."""
    import kv_cache_compression_anchor_amd as cg
    w = synth.workload(name)
    sel = list(w.selection())
    k, v = synth.gen_kv(w)
    kd, vd = gu.to_dev(k), gu.to_dev(v)
    tab = gu.gpu_tables(w, kd, vd)
    t = gu.torch()
    outs = [t.empty(cg.cg_encode_bound(tab, c), dtype=t.uint8, device="cuda") for c in range(len(sel))]
    sizes = cg.cg_encode_batch(tab, kd, vd, list(range(len(sel))), sel, outs)
    dblobs = [o[:n] for o, n in zip(outs, sizes)]
    del kd, vd
    ot = oracle.build_tables(oracle.params_for(w), k, v)
    oblobs = [oracle.encode_chunk(ot, k, v, c, q) for c, q in enumerate(sel)]
    P = 16
    table, n_pages = perm_table(k.shape[1], P, spare=16, seed=21)
    check(k.shape, tab, ot, dblobs, oblobs, [list(range(len(sel)))], P, table, n_pages)
