"""Pin the oracle's backward with central finite differences (fp64, brute force).

Every gradient the oracle returns -- dq, dk, dv, dbias and the sink gradient
-- is compared against central differences of the oracle's own forward on
tiny shapes, where the cap is strongly active (|u|/c up to ~3), with packed
segments, a causal sliding window, GQA, an additive bias and a learnable sink
all switched on together.  A dropped chain-rule term (the 1 - tanh^2 factor
of the soft-cap backward in "Support logits soft-capping in the Pallas-Triton
attention VJP"), a wrong sign in the sink gradient, or a transposed operand
fails here.
"""
import numpy as np
import pytest

from oracle import attention_backward, attention_forward


def _case(causal=True, window=5, segments=True, bias=True, sink="learnable", softcap=3.0, seed=0,
          k_start=False, dense=False):
    rng = np.random.default_rng(seed)
    B, S, Hq, Hkv, D = 2, 11, 4, 2, 6
    q = rng.standard_normal((B, S, Hq, D)) * 3.0
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    do = rng.standard_normal((B, S, Hq, D))
    kw = dict(causal=causal, window=window, softcap=softcap)
    if segments:
        kw["segment_ids"] = np.array([[0] * 4 + [1] * 7, [0] * 6 + [1] * 3 + [2] * 2])
    if bias:
        kw["bias"] = rng.standard_normal((B, Hq, S, S)) * 0.7
    if k_start:
        kw["k_start"] = np.array([[0, 0, 1, 1, 3, 3, 3, 5, 6, 6, 8], [0, 1, 1, 2, 2, 4, 4, 4, 7, 9, 9]])
    if dense:
        m = rng.random((B, S, S)) < 0.5
        m[:, np.arange(S), np.arange(S)] = True
        kw["mask"] = m
    if sink == "learnable":
        kw["sink"] = rng.standard_normal(Hq) * 2.0
    elif sink == "off_by_one":
        kw["sink"] = np.zeros(Hq)
    return q, k, v, do, kw


def _loss(q, k, v, do, kw):
    out, _ = attention_forward(q, k, v, **kw)
    return float((out * do).sum())


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


CASES = {
    "all_features": dict(),
    "plain_causal_cap": dict(window=0, segments=False, bias=False, sink=None),
    "nocausal_window_offbyone": dict(causal=False, window=4, segments=False, sink="off_by_one"),
    "nocap_sink_bias": dict(softcap=0.0, window=0),
    "k_start_cap_bias_sink": dict(window=0, segments=False, k_start=True),
    "dense_mask_cap_bias_sink": dict(causal=False, window=0, segments=False, dense=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_gradients_match_central_differences(name):
    q, k, v, do, kw = _case(**CASES[name])
    dq, dk, dv, dbias, dsink = attention_backward(q, k, v, do, **kw)
    loss = lambda: _loss(q, k, v, do, kw)  # noqa: E731
    assert _rel(dq, _fd(loss, q)) < 1e-7
    assert _rel(dk, _fd(loss, k)) < 1e-7
    assert _rel(dv, _fd(loss, v)) < 1e-7
    if "bias" in kw:
        assert _rel(dbias, _fd(loss, kw["bias"])) < 1e-7
    if "sink" in kw and CASES[name].get("sink", "learnable") == "learnable":
        assert _rel(dsink, _fd(loss, kw["sink"])) < 1e-7


def test_cap_is_active_in_the_fd_case():
    """The FD case must exercise the nonlinear part of the cap."""
    q, k, v, do, kw = _case()
    u = np.einsum("bihd,bjhd->bhij", q[:, :, :2], np.repeat(k, 2, axis=2)[:, :, :2]) / np.sqrt(6)
    assert np.max(np.abs(u)) / kw["softcap"] > 1.5


def test_gradients_where_the_cap_saturates():
    """Cap 30 with pre-cap logits reaching 168 (the tokamax page's check).

    tanh(168/30) is within 1e-4 of 1, so the chain factor 1 - t^2 is ~5e-5
    on the largest logits; the gradients must still match central
    differences (the factor is taken from the unmasked logit, never from a
    masked value).
    """
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))["cap_active"]
    rng = np.random.default_rng(21)
    B, S, H, D = 1, 9, 2, 4
    q = rng.standard_normal((B, S, H, D))
    k = rng.standard_normal((B, S, H, D))
    v = rng.standard_normal((B, S, H, D))
    do = rng.standard_normal((B, S, H, D))
    u = np.einsum("bihd,bjhd->bhij", q, k) / np.sqrt(D)
    q *= g["max_precap_logit"] / np.max(np.abs(np.tril(u[0, 0])))
    kw = dict(causal=True, softcap=g["softcap"])
    dq, dk, dv, _, _ = attention_backward(q, k, v, do, **kw)
    loss = lambda: _loss(q, k, v, do, kw)  # noqa: E731
    for grad, x in ((dq, q), (dk, k), (dv, v)):
        assert _rel(grad, _fd(loss, x, h=1e-6)) < 1e-6


@pytest.mark.parametrize("shape", [(1, 4), (2, 1), (1, 1)])
def test_broadcast_bias_gradient_matches_central_differences(shape):
    """A bias broadcast over batch rows and/or heads: its gradient, of the bias's own
    shape, against central differences taken on that small tensor."""
    q, k, v, do, kw = _case()
    rng = np.random.default_rng(7)
    kw["bias"] = rng.standard_normal(shape + (11, 11)) * 0.7
    dbias = attention_backward(q, k, v, do, **kw)[3]
    assert dbias.shape == kw["bias"].shape
    loss = lambda: _loss(q, k, v, do, kw)  # noqa: E731
    assert _rel(dbias, _fd(loss, kw["bias"])) < 1e-7
