"""The token rows the encoder (k_encode) and the histogram (k_histogram) load
ahead of use, replayed on the CPU for every chunk geometry of the five
workloads and for edge chunk sizes.  Both kernels pass the row as the raw
buffer load's scalar offset, which the buffer's range check does not cover, so
every row they name must lie inside the chunk; and a group that is coded or
counted must use the rows loaded for that group (a clamped prefetch is never
consumed).

The replays follow the kernels' loops statement for statement: loads of whole
groups of size GS = 10 two groups ahead (encoder: one wave, pairs of groups;
histogram: four waves taking every fourth group, two of their groups ahead),
a prefetch of a group past the last full one re-reading the last full group,
then the remaining groups (the last partial one) loaded directly."""
import pytest

import synth

GS = 10


def encoder_rows(tc):
    """(rows loaded, [(group coded, group its data was loaded for)])"""
    rows, used = [], []
    nfull = tc // GS
    ng = (tc + GS - 1) // GS
    g = 0
    if nfull > 0:
        def load(gg):
            gl = min(gg, nfull - 1)
            rows.extend(gl * GS + j for j in range(GS))
            return gl
        xa = load(0)
        xb = load(1)
        while g + 2 <= nfull:
            used.append((g, xa))
            xa = load(g + 2)
            used.append((g + 1, xb))
            xb = load(g + 3)
            g += 2
        if g < nfull:
            used.append((g, xa))
            g += 1
    while g < ng:
        ta = g * GS
        rows.extend(ta + j for j in range(min(GS, tc - ta)))
        used.append((g, g))
        g += 1
    return rows, used


def histogram_rows(tc, wave):
    rows, used = [], []
    nfull = tc // GS
    ng = (tc + GS - 1) // GS
    g = wave
    if nfull > 0:
        def load(gg):
            gl = min(gg, nfull - 1)
            rows.extend(gl * GS + j for j in range(GS))
            return gl
        xa = load(g)
        xb = load(g + 4)
        while g + 4 < nfull:
            used.append((g, xa))
            xa = load(g + 8)
            used.append((g + 4, xb))
            xb = load(g + 12)
            g += 8
        if g < nfull:
            used.append((g, xa))
            g += 4
    while g < ng:
        ta = g * GS
        rows.extend(ta + j for j in range(min(GS, tc - ta)))
        used.append((g, g))
        g += 4
    return rows, used


def chunk_sizes():
    sizes = set(range(1, 130)) | {1535, 1536, 1537, 65536}
    for name in synth.WORKLOADS:
        w = synth.workload(name)
        for ch in range(w.n_chunks):
            sizes.add(min(w.chunk_tokens, w.tokens - ch * w.chunk_tokens))
    return sorted(sizes)


@pytest.mark.parametrize("tc", chunk_sizes())
def test_encoder_prefetch_stays_inside_the_chunk(tc):
    rows, used = encoder_rows(tc)
    assert all(0 <= r < tc for r in rows), (tc, max(rows))
    ng = (tc + GS - 1) // GS
    assert [g for g, _ in used] == list(range(ng))
    assert all(g == src for g, src in used)


@pytest.mark.parametrize("tc", chunk_sizes())
def test_histogram_prefetch_stays_inside_the_chunk(tc):
    ng = (tc + GS - 1) // GS
    seen = []
    for wave in range(4):
        rows, used = histogram_rows(tc, wave)
        assert all(0 <= r < tc for r in rows), (tc, wave, max(rows))
        assert all(g == src for g, src in used)
        seen += [g for g, _ in used]
    assert sorted(seen) == list(range(ng))


def test_without_the_clamp_the_last_chunks_would_read_past_it():
    """The replay notices the hazard it guards against: with the clamp taken
    out, a 1536-token chunk's last prefetches name rows past the chunk."""
    tc, nfull = 1536, 1536 // GS
    assert (nfull + 1) * GS + GS - 1 >= tc  # the encoder's last prefetch, g + 3 = nfull + 1
    assert (nfull - 1 + 12) * GS >= tc       # the histogram's, up to g + 12
