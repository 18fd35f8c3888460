"""Host-side check of the dU hand-off between the dk/dv and dq kernels.

The dk/dv kernel stores dU in blocks (one per head, 32-key block and 32-query
block; in 16-bit two 1 KiB halves of 16 keys each, in fp32 one 4 KiB block
written by one 32-key group) and the dq kernel reads a block whenever some
query of its 32-query tile sees some key of the 32-key block.  This test walks
the store rule of the dk/dv kernels (16-bit: 32-key waves at D = 64, 16-key
waves, 8 per workgroup, 64-query items at D = 128; fp32: 1, 2 or 4 groups of
32 keys per workgroup and 32-query items, both halves of a block from its
group) and the read rule of the dq kernel over ragged causal / windowed / full
masks and checks that every store lands inside the workspace region, no half
is stored twice, and every half the dq kernel reads has been stored.  No GPU
needed.
"""
import numpy as np
import pytest


def visible_queries(j, Sq, causal, window, ks=None):
    """Queries that see key j: an interval [lo, hi) (Sq == Sk when causal).  ks: a non-decreasing
    k_start (query i sees keys j >= ks[i]), whose queries for key j end at the first ks above j."""
    lo, hi = (j, Sq) if causal else (0, Sq)
    if window > 0:
        if causal:
            hi = min(hi, j + window)
        else:
            lo, hi = max(lo, j - window + 1), min(hi, j + window)
    if ks is not None:
        hi = min(hi, int(np.searchsorted(ks, j, side="right")))
    return lo, max(hi, lo)


def stores(B, Hq, Hkv, Sq, Sk, causal, window, keys_per_wave, nw, bmq, ks=None):
    """Yield (b, hq, key block, query block, half) for every dU store."""
    G = Hq // Hkv
    bnk = keys_per_wave * nw
    for b in range(B):
        for hk in range(Hkv):
            for kb in range((Sk + bnk - 1) // bnk):
                k0 = kb * bnk
                lo_first, _ = visible_queries(k0, Sq, causal, window, ks)
                _, hi_last = visible_queries(min(k0 + bnk, Sk) - 1, Sq, causal, window, ks)
                qbeg = (lo_first // bmq) * bmq
                nqt = (hi_last - qbeg + bmq - 1) // bmq if hi_last > qbeg else 0
                for it in range(G * nqt):
                    hq = hk * G + it % G
                    q0 = qbeg + (nqt - 1 - it // G) * bmq
                    for w in range(nw):
                        kw = k0 + keys_per_wave * w
                        if keys_per_wave == 32:
                            if kw < Sk:
                                for half in (0, 1):
                                    yield b, hq, kw // 32, q0 // 32, half
                        elif k0 + 16 * (w & ~1) < Sk:
                            for kc in range(bmq // 32):
                                if kc == 0 or q0 + 32 * kc < Sq:
                                    yield b, hq, kw // 32, q0 // 32 + kc, w & 1


def reads(B, Hq, Sq, Sk, causal, window):
    for b in range(B):
        for hq in range(Hq):
            for qb in range((Sq + 31) // 32):
                qs = range(qb * 32, min(qb * 32 + 32, Sq))
                for kb in range((Sk + 31) // 32):
                    keys = range(kb * 32, min(kb * 32 + 32, Sk))
                    if any(visible_queries(j, Sq, causal, window)[0] <= q < visible_queries(j, Sq, causal, window)[1]
                           for j in keys for q in qs):
                        yield b, hq, kb, qb, 0
                        yield b, hq, kb, qb, 1


def keys_of(i, Sk, causal, window, ks=None):
    """The kernels' key interval [lo, hi) of query i: a query that sees no key gets an empty
    interval at lo == hi, clamped into [0, Sk] (with k_start it can lie beyond i itself)."""
    lo, hi = 0, Sk
    if ks is not None:
        lo = int(ks[i])
    if causal:
        hi = min(hi, i + 1)
    if window > 0:
        lo = max(lo, i - window + 1)
        if not causal:
            hi = min(hi, i + window)
    lo = min(lo, Sk)
    return lo, max(hi, lo)


def kernel_reads(B, Hq, Sq, Sk, causal, window, ks=None):
    """The dq kernels' read rule: a wave of 32 queries reads the block of keys kb32 .. + 31 when
    one of its queries has a non-empty key interval that meets the block (a wave vote)."""
    for b in range(B):
        for hq in range(Hq):
            for qb in range((Sq + 31) // 32):
                iv = [keys_of(q, Sk, causal, window, ks) for q in range(32 * qb, min(32 * qb + 32, Sq))]
                for kb in range((Sk + 31) // 32):
                    kb32 = 32 * kb
                    if kb32 < Sk and any(lo < hi and lo < kb32 + 32 and hi > kb32 for lo, hi in iv):
                        yield b, hq, kb, qb, 0
                        yield b, hq, kb, qb, 1


CASES = [(200, True, 0), (200, False, 0), (97, True, 0), (333, True, 50), (333, False, 40), (64, True, 0),
         (1, True, 0), (129, False, 0), (161, True, 16)]


@pytest.mark.parametrize("S,causal,window", CASES)
@pytest.mark.parametrize("keys_per_wave,nw,bmq", [(32, 4, 32), (16, 8, 64), (16, 4, 32), (32, 1, 32), (32, 2, 32)])
def test_du_blocks_cover_dq_reads(S, causal, window, keys_per_wave, nw, bmq):
    B, Hq, Hkv = 1, 4, 2
    nkb32, nqb32 = (S + 31) // 32, (S + 31) // 32
    seen = set()
    for b, hq, kb, qb, half in stores(B, Hq, Hkv, S, S, causal, window, keys_per_wave, nw, bmq):
        assert 0 <= kb < nkb32 and 0 <= qb < nqb32, (kb, qb)
        key = (b, hq, kb, qb, half)
        assert key not in seen, f"half stored twice: {key}"
        seen.add(key)
    missing = [r for r in reads(B, Hq, S, S, causal, window) if r not in seen]
    assert not missing, f"dq reads unwritten halves, e.g. {missing[:3]}"


# Sq != Sk (no causal mask): with Sq > Sk and a window the last queries see no key, whole
# 32-query waves of them when Sk + window falls far enough below Sq; their empty intervals sit
# at Sk, inside a 32-key block when Sk is not a multiple of 32, and dk/dv writes no block for
# them, so the kernels' read rule must treat an empty interval as no keys at all.
CROSS = [(252, 56, 47), (184, 59, 42), (171, 89, 38), (96, 32, 40), (100, 181, 60), (160, 181, 60),
         (129, 70, 0), (300, 33, 5)]


@pytest.mark.parametrize("Sq,Sk,window", CROSS)
@pytest.mark.parametrize("keys_per_wave,nw,bmq", [(32, 4, 32), (16, 8, 64), (16, 8, 32), (32, 1, 32), (32, 2, 32)])
def test_du_blocks_cover_the_kernels_reads_across_lengths(Sq, Sk, window, keys_per_wave, nw, bmq):
    B, Hq, Hkv = 1, 2, 1
    nkb32, nqb32 = (Sk + 31) // 32, (Sq + 31) // 32
    seen = set()
    for b, hq, kb, qb, half in stores(B, Hq, Hkv, Sq, Sk, False, window, keys_per_wave, nw, bmq):
        assert 0 <= kb < nkb32 and 0 <= qb < nqb32, (kb, qb)
        key = (b, hq, kb, qb, half)
        assert key not in seen, f"half stored twice: {key}"
        seen.add(key)
    ideal = set(reads(B, Hq, Sq, Sk, False, window))
    got = set(kernel_reads(B, Hq, Sq, Sk, False, window))
    assert ideal <= got, "the read rule skips a block holding a visible pair"
    missing = sorted(r for r in got if r not in seen)
    assert not missing, f"dq reads unwritten halves, e.g. {missing[:3]}"


@pytest.mark.parametrize("S,causal,window", CASES)
def test_kernel_read_rule_equals_the_ideal_one_at_equal_lengths(S, causal, window):
    assert set(kernel_reads(1, 1, S, S, causal, window)) == set(reads(1, 1, S, S, causal, window))


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("keys_per_wave,nw,bmq", [(32, 4, 32), (16, 8, 64), (16, 8, 32), (32, 1, 32)])
def test_du_blocks_cover_the_kernels_reads_with_k_start(seed, keys_per_wave, nw, bmq):
    """Causal with a random non-decreasing k_start: queries with k_start above their own position
    see no key, and their empty intervals sit at k_start, beyond them."""
    rng = np.random.default_rng(seed)
    S = int(rng.integers(40, 300))
    ks = np.sort(rng.integers(0, S + 1, size=S))
    seen = set(stores(1, 2, 1, S, S, True, 0, keys_per_wave, nw, bmq, ks))
    got = set(kernel_reads(1, 2, S, S, True, 0, ks))
    missing = sorted(r for r in got if r not in seen)
    assert not missing, f"dq reads unwritten halves, e.g. {missing[:3]}"
