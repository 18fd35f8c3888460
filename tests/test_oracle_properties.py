"""Pin the oracle to closed forms, invariants and reductions (CPU, fp64).

Each test states a fact the mathematics fixes independently of how the
oracle is written:

* a worked example whose logits are chosen so that tanh takes exact values
  (atanh(1/2) = ln(3)/2), solved by hand;
* single-key rows, all-zero queries (uniform attention), the large-cap limit
  c*tanh(u/c) = u - u^3/(3c^2) + ..., the softmax normalisation with the sink
  column, and the sink-gradient identity -sum_i p_i <dO_i, o_i>;
* packing ("a packed batch equals its segments run alone, with zero leakage",
  MaxText commit message quoted on "Support logits soft-capping in the
  Pallas-Triton attention VJP"), GQA against repeated K/V, THD against
  segment ids, the sliding-window pair count, fully masked rows.
"""
import math

import numpy as np
import pytest

from oracle import attention_backward, attention_forward, visibility


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def _rand(B=2, S=24, Hq=4, Hkv=2, D=8, seed=0, qs=2.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, S, Hq, D)) * qs, rng.standard_normal((B, S, Hkv, D)),
            rng.standard_normal((B, S, Hkv, D)), rng.standard_normal((B, S, Hq, D)), rng)


# --------------------------------------------------------------- worked example

@pytest.mark.parametrize("off_by_one", [False, True])
def test_hand_worked_capped_example(off_by_one):
    """c=2, D=1, scale=1: logits ln3, -ln3, 0 are capped to exactly 1, -1, 0.

    tanh(ln(3)/2) = (3-1)/(3+1) = 1/2, so s = c*t = (1, -1, 0) and the cap
    factors 1 - t^2 are (3/4, 3/4, 1).  With values (1, 2, 4), dO = 1 and an
    optional off-by-one sink (logit 0, one extra column):
      Z = e + 1/e + 1 (+1),  P = (e, 1/e, 1)/Z,  o = (e + 2/e + 4)/Z,
      lse = ln Z,  dv = P,  dU_j = P_j (v_j - o) f_j,  dq = sum_j dU_j k_j,
      dk_j = dU_j q,  dbias_j = dU_j,  dsink = -p o with p = 1/Z.
    """
    L3 = math.log(3.0)
    q = np.array([[[[1.0]]]])
    k = np.array([[[[L3]], [[-L3]], [[0.0]]]])
    v = np.array([[[[1.0]], [[2.0]], [[4.0]]]])
    bias = np.zeros((1, 1, 1, 3))
    e = math.e
    Z = e + 1 / e + 1 + (1.0 if off_by_one else 0.0)
    P = np.array([e, 1 / e, 1.0]) / Z
    o = (e + 2 / e + 4) / Z
    f = np.array([0.75, 0.75, 1.0])
    dU = P * (np.array([1.0, 2.0, 4.0]) - o) * f
    kw = dict(softcap=2.0, scale=1.0, bias=bias, sink=np.zeros(1) if off_by_one else None)
    # the oracle's key axis is 3 keys for one query: build Sq=1, Sk=3 (non-causal)
    out, lse = attention_forward(q, k, v, **kw)
    assert abs(out[0, 0, 0, 0] - o) < 1e-14
    assert abs(lse[0, 0, 0] - math.log(Z)) < 1e-14
    dq, dk, dv, dbias, dsink = attention_backward(q, k, v, np.ones_like(q), **kw)
    assert np.max(np.abs(dv[0, :, 0, 0] - P)) < 1e-14
    assert abs(dq[0, 0, 0, 0] - float((dU * np.array([L3, -L3, 0.0])).sum())) < 1e-14
    assert np.max(np.abs(dk[0, :, 0, 0] - dU)) < 1e-14
    assert np.max(np.abs(dbias[0, 0, 0] - dU)) < 1e-14
    if off_by_one:
        assert abs(dsink[0] + o / Z) < 1e-14


# --------------------------------------------------------------- special cases

@pytest.mark.parametrize("softcap", [0.0, 5.0])
def test_window_of_one_copies_values(softcap):
    """W = 1: every row sees only its own key, so o_i = v_i and dq = dk = 0."""
    q, k, v, do, _ = _rand()
    out, lse = attention_forward(q, k, v, causal=True, window=1, softcap=softcap)
    G = 2
    assert np.max(np.abs(out - np.repeat(v, G, axis=2))) < 1e-14
    dq, dk, dv, _, _ = attention_backward(q, k, v, do, causal=True, window=1, softcap=softcap)
    assert np.max(np.abs(dq)) < 1e-14 and np.max(np.abs(dk)) < 1e-14
    assert np.max(np.abs(dv - do.reshape(2, 24, 2, G, 8).sum(axis=3))) < 1e-14


def test_first_causal_row_with_sink_is_a_sigmoid():
    """Row 0 sees only key 0: o_0 = sigmoid(s_00 - sigma) v_0.

    Pick q_0 = k_0 * (c * atanh(1/2) * sqrt(D) / |k_0|^2) so that u_00 =
    c*atanh(1/2) and s_00 = c/2 exactly.
    """
    c, D = 4.0, 8
    q, k, v, do, rng = _rand(B=1, S=5, Hq=1, Hkv=1, D=D)
    k0 = k[0, 0, 0]
    q[0, 0, 0] = k0 * (c * math.atanh(0.5) * math.sqrt(D) / float(k0 @ k0))
    sigma = 0.7
    out, lse = attention_forward(q, k, v, causal=True, softcap=c, sink=np.array([sigma]))
    p = 1.0 / (1.0 + math.exp(-(c / 2 - sigma)))
    assert np.max(np.abs(out[0, 0, 0] - p * v[0, 0, 0])) < 1e-13
    assert abs(lse[0, 0, 0] - math.log(math.exp(c / 2) + math.exp(sigma))) < 1e-13


@pytest.mark.parametrize("softcap", [0.0, 7.0])
def test_zero_queries_average_the_visible_values(softcap):
    """q = 0 and no bias: u = 0, tanh(0) = 0, attention is uniform."""
    q, k, v, do, _ = _rand(B=1, Hq=2, Hkv=1)
    q[:] = 0.0
    out, _ = attention_forward(q, k, v, causal=True, softcap=softcap)
    ref = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, 25)[:, None]
    assert np.max(np.abs(out[0, :, 0] - ref)) < 1e-14
    assert np.max(np.abs(out[0, :, 1] - ref)) < 1e-14


def test_large_cap_converges_quadratically_to_plain_attention():
    """c*tanh(u/c) = u - u^3/(3c^2) + O(c^-4): error falls 100x per 10x in c."""
    q, k, v, do, _ = _rand(seed=4, qs=3.0)
    plain, _ = attention_forward(q, k, v, causal=True)
    e1 = np.max(np.abs(attention_forward(q, k, v, causal=True, softcap=300.0)[0] - plain))
    e2 = np.max(np.abs(attention_forward(q, k, v, causal=True, softcap=3000.0)[0] - plain))
    assert 1e-8 < e2 < e1
    assert 95.0 < e1 / e2 < 105.0
    g1 = attention_backward(q, k, v, do, causal=True, softcap=300.0)[0]
    g2 = attention_backward(q, k, v, do, causal=True, softcap=3000.0)[0]
    g0 = attention_backward(q, k, v, do, causal=True)[0]
    r = np.max(np.abs(g1 - g0)) / np.max(np.abs(g2 - g0))
    assert 95.0 < r < 105.0


def test_cap_bounds_the_logits():
    """|c*tanh(u/c)| < c: an enormous logit cannot take more than e^c/(e^c + 2e^-c).

    v holds one-hot rows, so the output of row 2 is its probability vector.
    """
    q, k, v, do, _ = _rand(B=1, S=3, Hq=1, Hkv=1, D=3, qs=1.0)
    q[0, 2, 0] = k[0, 0, 0] * 1e6          # u_20 enormous and positive
    v[0, :, 0] = np.eye(3)
    c = 1.0
    out, lse = attention_forward(q, k, v, causal=True, softcap=c)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert lse[0, 0, 2] < c + math.log(3) + 1e-12
    assert out[0, 2, 0, 0] <= math.exp(c) / (math.exp(c) + 2 * math.exp(-c)) + 1e-15
    assert out[0, 2, 0, 1] >= math.exp(-c) / (3 * math.exp(c)) - 1e-15


# --------------------------------------------------------------- invariants

@pytest.mark.parametrize("sink", [None, "learnable"])
def test_rows_and_sink_probability_sum_to_one(sink):
    """With v = 1, o_i = sum_j P_ij = 1 - p_i where p_i = exp(sigma - lse_i)."""
    q, k, v, do, rng = _rand(seed=6)
    v[:] = 1.0
    s = rng.standard_normal(4) * 5 if sink else None
    seg = np.array([[0] * 9 + [1] * 15, [0] * 24])
    out, lse = attention_forward(q, k, v, causal=True, window=7, softcap=3.0, segment_ids=seg, sink=s)
    p = np.zeros_like(lse) if s is None else np.exp(s[None, :, None] - lse)
    total = out[..., 0] + p.transpose(0, 2, 1)
    assert np.max(np.abs(total - 1.0)) < 1e-14


def test_sink_gradient_identity():
    """dsink_h = -sum_{b,i} exp(sigma_h - lse_bhi) <dO_bih, o_bih>."""
    q, k, v, do, rng = _rand(seed=7)
    s = rng.standard_normal(4) * 5
    kw = dict(causal=True, softcap=3.0, sink=s)
    out, lse = attention_forward(q, k, v, **kw)
    *_, dsink = attention_backward(q, k, v, do, **kw)
    delta = np.einsum("bihd,bihd->bhi", do, out)
    ref = -np.sum(np.exp(s[None, :, None] - lse) * delta, axis=(0, 2))
    assert _rel(dsink, ref) < 1e-13


def test_packed_batch_equals_segments_run_alone():
    q, k, v, do, rng = _rand(B=1, S=30, seed=8)
    bias = rng.standard_normal((1, 4, 30, 30))
    sink = rng.standard_normal(4)
    cuts = [0, 7, 19, 30]
    seg = np.zeros((1, 30), dtype=int)
    for n in range(3):
        seg[0, cuts[n]:cuts[n + 1]] = n
    kw = dict(causal=True, window=6, softcap=2.5, sink=sink)
    out, lse = attention_forward(q, k, v, segment_ids=seg, bias=bias, **kw)
    dq, dk, dv, dbias, dsink = attention_backward(q, k, v, do, segment_ids=seg, bias=bias, **kw)
    dsink_sum = np.zeros(4)
    for n in range(3):
        r = slice(cuts[n], cuts[n + 1])
        o2, l2 = attention_forward(q[:, r], k[:, r], v[:, r], bias=bias[:, :, r, r], **kw)
        g = attention_backward(q[:, r], k[:, r], v[:, r], do[:, r], bias=bias[:, :, r, r], **kw)
        assert np.max(np.abs(out[:, r] - o2)) < 1e-14
        assert np.max(np.abs(lse[:, :, r] - l2)) < 1e-14
        for a, b in zip((dq[:, r], dk[:, r], dv[:, r], dbias[:, :, r, r]), g[:4]):
            assert np.max(np.abs(a - b)) < 1e-13
        dsink_sum += g[4]
    assert np.max(np.abs(dsink - dsink_sum)) < 1e-13
    # no leakage: dbias across segments is exactly zero
    cross = seg[0][:, None] != seg[0][None, :]
    assert np.all(dbias[0][:, cross] == 0.0)


def test_perturbing_one_segment_leaves_the_others_bit_identical():
    q, k, v, do, rng = _rand(B=1, S=30, seed=9)
    seg = np.array([[0] * 13 + [1] * 17])
    kw = dict(causal=True, softcap=4.0, segment_ids=seg)
    o1, _ = attention_forward(q, k, v, **kw)
    g1 = attention_backward(q, k, v, do, **kw)
    k2, v2 = k.copy(), v.copy()
    k2[:, :13] += 3.0
    v2[:, :13] -= 1.0
    o2, _ = attention_forward(q, k2, v2, **kw)
    g2 = attention_backward(q, k2, v2, do, **kw)
    assert np.array_equal(o1[:, 13:], o2[:, 13:])
    for a, b in zip(g1[:3], g2[:3]):
        assert np.array_equal(a[:, 13:], b[:, 13:])


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v, do, rng = _rand(Hq=6, Hkv=2, seed=10)
    sink = rng.standard_normal(6)
    kw = dict(causal=True, softcap=3.0, window=9, sink=sink)
    out, lse = attention_forward(q, k, v, **kw)
    kr, vr = np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2)
    out2, lse2 = attention_forward(q, kr, vr, **kw)
    assert np.max(np.abs(out - out2)) < 1e-14 and np.max(np.abs(lse - lse2)) < 1e-14
    dq, dk, dv, _, ds = attention_backward(q, k, v, do, **kw)
    dq2, dk2, dv2, _, ds2 = attention_backward(q, kr, vr, do, **kw)
    assert np.max(np.abs(dq - dq2)) < 1e-13
    assert np.max(np.abs(dk - dk2.reshape(2, 24, 2, 3, 8).sum(3))) < 1e-13
    assert np.max(np.abs(dv - dv2.reshape(2, 24, 2, 3, 8).sum(3))) < 1e-13
    assert np.max(np.abs(ds - ds2)) < 1e-13


def test_thd_with_cu_seqlens_equals_segment_ids():
    q, k, v, do, rng = _rand(B=1, S=40, seed=11)
    cu = np.array([0, 9, 10, 33, 40])
    seg = np.zeros((1, 40), dtype=int)
    for n in range(4):
        seg[0, cu[n]:cu[n + 1]] = n
    kw = dict(causal=True, softcap=3.0)
    o1, l1 = attention_forward(q, k, v, segment_ids=seg, **kw)
    o2, l2 = attention_forward(q[0], k[0], v[0], cu_seqlens=cu, **kw)
    assert np.array_equal(o1[0], o2) and np.array_equal(l1[0], l2)
    g1 = attention_backward(q, k, v, do, segment_ids=seg, **kw)
    g2 = attention_backward(q[0], k[0], v[0], do[0], cu_seqlens=cu, **kw)
    for a, b in zip(g1[:3], g2[:3]):
        assert np.array_equal(a[0], b)


def test_window_at_least_the_length_is_plain_causal():
    q, k, v, do, _ = _rand(seed=12)
    a = attention_forward(q, k, v, causal=True, softcap=3.0)[0]
    b = attention_forward(q, k, v, causal=True, softcap=3.0, window=24)[0]
    assert np.array_equal(a, b)


def test_sliding_window_pair_count():
    """Causal window W keeps exactly min(i+1, W) keys in row i."""
    S, W = 8192, 1024
    total = 0
    for r0 in range(0, S, 1024):
        total += int(visibility(S, S, True, W, rows=slice(r0, r0 + 1024)).sum())
    assert total == sum(min(i + 1, W) for i in range(S)) == 7864832
    assert int(visibility(S, S, True, 0, rows=slice(S - 1, S)).sum()) == S


def test_fully_masked_rows():
    """A row with no visible key: o = 0, lse = -inf; with a sink p = 1, lse = sigma."""
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, 10, 1, 4))
    k = rng.standard_normal((1, 3, 1, 4))
    v = rng.standard_normal((1, 3, 1, 4))
    do = rng.standard_normal((1, 10, 1, 4))
    out, lse = attention_forward(q, k, v, window=2)          # rows >= 4 see nothing
    assert np.all(out[0, 4:] == 0.0) and np.all(np.isneginf(lse[0, 0, 4:]))
    dq, dk, dv, _, _ = attention_backward(q, k, v, do, window=2)
    assert np.all(dq[0, 4:] == 0.0)
    out, lse = attention_forward(q, k, v, window=2, sink=np.array([0.3]))
    assert np.all(out[0, 4:] == 0.0) and np.allclose(lse[0, 0, 4:], 0.3, atol=1e-15)
