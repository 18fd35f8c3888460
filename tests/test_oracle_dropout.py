"""Pins of the oracle's dropout: its generator and the dropout arithmetic.

* Philox4x32-10 against the known-answer vectors published with the
  generator's reference implementation (Random123, the code that accompanies
  "Parallel random numbers: as easy as 1, 2, 3"): zero counter and key, all
  ones, and the digits-of-pi counter and key.
* The keep fraction of many draws is 1 - p within binomial error, for each
  of the eight 16-bit halves of an evaluation separately; halves of the same
  word and of different words decide independently (a wrong half or word
  selection would repeat or correlate decisions); the threshold is
  floor(p 2^16), so p = 0 and p below 2^-16 keep everything.
* The gradients of the dropped forward, with the keep decisions held fixed,
  equal central differences (cap, bias, learnable sink, segments active).
* Dropout is unbiased: the mean output over many seeds is the undropped one.
"""
import numpy as np
import pytest

from oracle import attention_backward, attention_forward, group_backward, group_forward
from oracle.philox import drop_probability, dropout_keep, philox4x32_10, threshold

KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    got = philox4x32_10(*ctr, *key)
    assert tuple(int(x) for x in got) == want


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_fraction_is_one_minus_p(p):
    n_rows, Sk = 512, 2048
    keep = dropout_keep(1, 3, 8, np.arange(n_rows), Sk, p, seed=1234567891011, offset=77)
    frac = keep.mean()
    sigma = np.sqrt(p * (1 - p) / keep.size)
    assert abs(frac - (1 - p)) < 5 * sigma
    # different heads, rows, seeds and offsets draw different decisions
    other = dropout_keep(1, 4, 8, np.arange(n_rows), Sk, p, seed=1234567891011, offset=77)
    assert (keep != other).mean() > 0.1


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_each_half_keeps_one_minus_p_and_halves_are_independent(p):
    n_rows, Sk = 256, 4096
    keep = dropout_keep(0, 1, 4, np.arange(n_rows), Sk, p, seed=0xDEADBEEF12345, offset=5)
    q = 1 - drop_probability(p)
    by_half = keep.reshape(n_rows, Sk // 8, 8)
    n = by_half[..., 0].size
    for m in range(8):
        assert abs(by_half[..., m].mean() - q) < 5 * np.sqrt(q * (1 - q) / n), m
    # two halves of one word (m, m + 1), and halves of different words (m, m + 2), (m, m + 4)
    for a, c in ((0, 1), (2, 3), (6, 7), (0, 2), (1, 5), (3, 4)):
        both = (by_half[..., a] & by_half[..., c]).mean()
        assert abs(both - q * q) < 5 * np.sqrt(q * q * (1 - q * q) / n), (a, c)


def test_threshold_is_p_rounded_down_to_sixteen_bits():
    assert threshold(0.1) == 6553 and drop_probability(0.1) == 6553 / 65536
    assert threshold(0.5) == 32768 and drop_probability(0.5) == 0.5
    assert threshold(1.0 - 2.0 ** -20) == 0xFFFF
    assert threshold(2.0 ** -17) == 0
    assert dropout_keep(0, 0, 1, np.arange(64), 256, 2.0 ** -17, seed=3, offset=0).all()


def test_zero_probability_keeps_everything_and_changes_nothing():
    assert threshold(0.0) == 0
    rng = np.random.default_rng(0)
    q, k, v, do = (rng.standard_normal(s) for s in ((2, 19, 4, 8), (2, 19, 2, 8), (2, 19, 2, 8), (2, 19, 4, 8)))
    a = attention_forward(q, k, v, causal=True, softcap=5.0) + attention_backward(q, k, v, do, causal=True, softcap=5.0)
    b = attention_forward(q, k, v, causal=True, softcap=5.0, dropout_p=0.0, dropout_seed=9) + \
        attention_backward(q, k, v, do, causal=True, softcap=5.0, dropout_p=0.0, dropout_seed=9)
    for x, y in zip(a, b):
        if x is not None:
            assert np.array_equal(x, y)


def _fd(fn, x, h=1e-5):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        fp = fn()
        x[idx] = old - h
        fm = fn()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def test_dropout_gradients_match_central_differences():
    rng = np.random.default_rng(3)
    S, G, D = 10, 2, 6
    q = rng.standard_normal((S, G, D)) * 3.0
    k = rng.standard_normal((S, D))
    v = rng.standard_normal((S, D))
    do = rng.standard_normal((S, G, D))
    bias = rng.standard_normal((G, S, S)) * 0.7
    sink = rng.standard_normal(G) * 2.0
    keep_all = rng.random((G, S, S)) > 0.4
    drop = (0.4, lambda g, rows: keep_all[g, rows])
    kw = dict(causal=True, softcap=3.0, seg=np.array([0] * 4 + [1] * 6), sink=sink, dropout=drop)

    def loss():
        o, _ = group_forward(q, k, v, bias=bias, **kw)
        return float((o * do).sum())

    dq, dk, dv, dbias, dsink = group_backward(q, k, v, do, bias=bias, **kw)
    assert _rel(dq, _fd(loss, q)) < 1e-7
    assert _rel(dk, _fd(loss, k)) < 1e-7
    assert _rel(dv, _fd(loss, v)) < 1e-7
    assert _rel(dbias, _fd(loss, bias)) < 1e-7
    assert _rel(dsink, _fd(loss, sink)) < 1e-7


@pytest.mark.parametrize("p", [0.5, 0.3])
def test_dropout_is_unbiased_over_seeds(p):
    """p = 0.3 is not a multiple of 2^-16: the scale 1 / (1 - p') of the rounded probability
    keeps the expectation exact."""
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal(s) for s in ((1, 8, 1, 4), (1, 8, 1, 4), (1, 8, 1, 4)))
    ref, _ = attention_forward(q, k, v, causal=True)
    acc = np.zeros_like(ref)
    n = 3000
    for seed in range(n):
        o, _ = attention_forward(q, k, v, causal=True, dropout_p=p, dropout_seed=seed)
        acc += o
    mean = acc / n
    # standard error of the mean: each output is a sum of at most 8 terms of size |P v| / (1 - p)
    assert _rel(mean, ref) < 0.06
