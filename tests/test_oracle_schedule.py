"""fp64 emulation of the fused kernel's tile schedule against the oracle.

The learnable-sink page ("learnable softmax sink with context-parallel p2p",
"What changed" and the FP64-emulation paragraph of "Verification") checks a
tiled schedule by emulating it in fp64: seeding the sink into every tile's
softmax statistics counts it once per visited tile and is wrong; seeding it
once per query row matches the plain result to rounding.  The same holds for
the single-GPU online softmax: the running (max, sum) of each query row is
seeded once with the sink and then merged over the visible key tiles.  This
emulation follows the forward kernel's order (query tiles, visible key-tile
range, skip of tiles outside it, online rescaling) in float64 and must agree
with the oracle to ~1e-13; the negative control (sink seeded per tile) must
not.
"""
import math

import numpy as np
import pytest

from oracle import attention_forward


def _emulate(q, k, v, causal, window, softcap, seg, sink, BM, BN, sink_per_tile=False):
    """Online-softmax forward over key tiles for one (b, head), fp64."""
    S, D = q.shape
    tau = 1.0 / math.sqrt(D)
    segid = np.zeros(S, int) if seg is None else seg
    start = np.array([np.searchsorted(segid, segid[i], "left") for i in range(S)])
    end = np.array([np.searchsorted(segid, segid[i], "right") for i in range(S)])
    lo = start.copy()
    hi = end.copy()
    if causal:
        hi = np.minimum(hi, np.arange(S) + 1)
    if window > 0:
        lo = np.maximum(lo, np.arange(S) - window + 1)
        if not causal:
            hi = np.minimum(hi, np.arange(S) + window)
    out = np.zeros_like(q)
    lse = np.zeros(S)
    for i0 in range(0, S, BM):
        i1 = min(S, i0 + BM)
        rows = np.arange(i0, i1)
        m = np.full(i1 - i0, -np.inf)
        l = np.zeros(i1 - i0)
        acc = np.zeros((i1 - i0, v.shape[1]))
        if sink is not None and not sink_per_tile:
            m[:] = sink
            l[:] = 1.0
        kt0 = (lo[i0] // BN) * BN
        for j0 in range(kt0, hi[i1 - 1], BN):
            j1 = min(S, j0 + BN)
            cols = np.arange(j0, j1)
            u = tau * q[rows] @ k[cols].T
            s = softcap * np.tanh(u / softcap) if softcap > 0 else u
            vis = (cols[None, :] >= lo[rows][:, None]) & (cols[None, :] < hi[rows][:, None])
            s = np.where(vis, s, -np.inf)
            tile_m = s.max(axis=1)
            if sink is not None and sink_per_tile:
                tile_m = np.maximum(tile_m, sink)
            m_new = np.maximum(m, tile_m)
            base = np.where(np.isfinite(m_new), m_new, 0.0)
            alpha = np.where(np.isfinite(m), np.exp(m - base), 0.0)
            p = np.where(vis, np.exp(s - base[:, None]), 0.0)
            l = l * alpha + p.sum(axis=1)
            if sink is not None and sink_per_tile:
                l += np.exp(sink - base)
            acc = acc * alpha[:, None] + p @ v[cols]
            m = m_new
        out[rows] = acc / l[:, None]
        lse[rows] = m + np.log(l)
    return out, lse


def _data(seed=0, S=97, D=16):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((S, D)) * 3, rng.standard_normal((S, D)), rng.standard_normal((S, D)))


CASES = [
    dict(causal=True, window=0, seg=None),
    dict(causal=True, window=20, seg=None),
    dict(causal=False, window=0, seg=None),
    dict(causal=True, window=0, seg=np.repeat([0, 1, 2, 3], [10, 33, 40, 14])),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("tiles", [(32, 32), (16, 64), (64, 16)])
def test_sink_seeded_once_matches_the_oracle(case, tiles):
    c = CASES[case]
    q, k, v = _data(case)
    sink = 1.7
    out_e, lse_e = _emulate(q, k, v, c["causal"], c["window"], 4.0, c["seg"], sink, *tiles)
    seg = None if c["seg"] is None else c["seg"][None]
    out, lse = attention_forward(q[None, :, None], k[None, :, None], v[None, :, None], causal=c["causal"],
                                 window=c["window"], softcap=4.0, segment_ids=seg, sink=np.array([sink]))
    assert np.max(np.abs(out_e - out[0, :, 0])) < 1e-13
    assert np.max(np.abs(lse_e - lse[0, 0])) < 1e-13


def test_sink_seeded_per_tile_is_wrong():
    """Negative control: with the sink in every tile's statistics the result drifts."""
    q, k, v = _data(4)
    sink = 1.7
    good, _ = _emulate(q, k, v, True, 0, 4.0, None, sink, 16, 16)
    bad, bad_lse = _emulate(q, k, v, True, 0, 4.0, None, sink, 16, 16, sink_per_tile=True)
    assert np.max(np.abs(good - bad)) > 1e-3
