"""Host-side check of who writes dbias on the bf16 path with D = 128 / 256.

The dk/dv kernel with a bias owns the dbias columns of its key block: its
items write whole (query tile x key block) tiles over the query rows
[qbeg, qbeg + nqt * BMQ) -- the visible value, or 0 at a masked pair -- and
afterwards it writes zeros on every other query row of those columns, on the
grounds that those rows see none of the block's keys.  This test walks that
rule over ragged causal / windowed / packed-segment / cross-length masks and
checks that every element of dbias is written, and that the zero rows hold
no visible pair (which is what the monotone visible query range of a key
guarantees).  With a bias broadcast over heads the same rows split the work
between two kernels: dk/dv writes the covered rows of its head-summed slab and
the slab reduction, recomputing [qbeg, qbeg + nqt * BMQ) per key block, reads
only those and writes the zeros of the others.  No GPU needed.
"""
import numpy as np
import pytest


def queries_of(j, Sq, causal, window, seg):
    """Queries that see key j: an interval [lo, hi), as the kernels compute it."""
    lo, hi = 0, Sq
    if seg is not None:
        s = seg[j]
        idx = np.nonzero(seg[:Sq] == s)[0]
        lo, hi = (int(idx[0]), int(idx[-1]) + 1) if len(idx) else (0, 0)
    if causal:
        lo = max(lo, j)
    if window > 0:
        hi = min(hi, j + window)
        if not causal:
            lo = max(lo, j - window + 1)
    lo = min(lo, Sq)
    return lo, max(hi, lo)


def visible(i, j, causal, window, seg):
    if seg is not None and seg[i] != seg[j]:
        return False
    if causal and j > i:
        return False
    if window > 0 and (i - j >= window if causal else abs(i - j) >= window):
        return False
    return True


def writers(Sq, Sk, causal, window, seg, bnk, bmq):
    """Per dbias element: 1 where a tile writes it, 2 where the zero fill does."""
    who = np.zeros((Sq, Sk), np.int8)
    for kb in range((Sk + bnk - 1) // bnk):
        k0, k1 = kb * bnk, min(kb * bnk + bnk, Sk)
        lo_first, _ = queries_of(k0, Sq, causal, window, seg)
        _, hi_last = queries_of(k1 - 1, Sq, causal, window, seg)
        qbeg = (lo_first // bmq) * bmq
        nqt = (hi_last - qbeg + bmq - 1) // bmq if hi_last > qbeg else 0
        z_lo = min(qbeg, Sq)
        z_hi = max(z_lo, min(qbeg + nqt * bmq, Sq))
        assert not who[z_lo:z_hi, k0:k1].any() and not who[:z_lo, k0:k1].any()
        who[z_lo:z_hi, k0:k1] = 1
        who[:z_lo, k0:k1] = 2
        who[z_hi:, k0:k1] = 2
    return who


def segments(S, cuts):
    seg = np.zeros(S, np.int32)
    for c in cuts:
        seg[c:] += 1
    return seg


CASES = [
    (300, 300, True, 0, None),
    (300, 300, False, 0, None),
    (333, 333, True, 50, None),
    (333, 333, False, 40, None),
    (161, 161, True, 16, None),
    (97, 97, True, 0, None),
    (400, 400, True, 0, [37, 130, 131, 250]),
    (400, 400, True, 64, [100, 333]),
    (200, 264, False, 0, None),
    (264, 200, False, 30, None),
    (1, 1, True, 0, None),
]


@pytest.mark.parametrize("Sq,Sk,causal,window,cuts", CASES)
@pytest.mark.parametrize("bnk,bmq", [(128, 32), (64, 32)])
def test_dbias_tiles_and_zero_rows_cover_every_element(Sq, Sk, causal, window, cuts, bnk, bmq):
    seg = None if cuts is None else segments(max(Sq, Sk), cuts)
    who = writers(Sq, Sk, causal, window, seg, bnk, bmq)
    assert (who > 0).all(), "dbias elements written by nobody"
    for i in range(Sq):
        for j in np.nonzero(who[i] == 2)[0]:
            assert not visible(i, int(j), causal, window, seg), f"zero fill over visible pair ({i}, {j})"
