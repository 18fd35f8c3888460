"""Pin the oracle to a library routine: PyTorch's scaled_dot_product_attention in fp64.

With the cap off (softcap = 0 is a no-op: "Thread tanh logit softcapping
through FlashAttention (FA2, opt-in FA3)", "What changed"), the oracle must be
plain softmax attention, so it must equal SDPA run on the CPU in float64 with
the visibility written as an additive mask and K/V repeated per query head.
The sink ("What changed" of the learnable-sink page: one more softmax
column) must equal SDPA with one extra key whose vector and value are zero and
whose additive mask is the sink logit.  Gradients are compared against
SDPA's own autograd backward.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention_backward, attention_forward


def _inputs(B=2, S=37, Hq=6, Hkv=3, D=16, seed=1):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S, Hq, D)) * 2
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    do = rng.standard_normal((B, S, Hq, D))
    return q, k, v, do, rng


def _mask(S, causal, window, seg):
    """Visibility written independently of the oracle (loops, tiny sizes)."""
    B = 1 if seg is None else seg.shape[0]
    m = np.zeros((B, 1, S, S), dtype=bool)
    for b in range(B):
        for i in range(S):
            for j in range(S):
                ok = True
                if causal and j > i:
                    ok = False
                if window > 0:
                    d = i - j
                    if causal and not (0 <= d < window):
                        ok = False
                    if not causal and abs(d) >= window:
                        ok = False
                if seg is not None and seg[b, i] != seg[b, j]:
                    ok = False
                m[b, 0, i, j] = ok
    return m


def _sdpa(q, k, v, mask_bool, bias=None, sink=None, scale=None, grad=False, do=None):
    G = q.shape[2] // k.shape[2]
    tq = torch.tensor(q, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(grad)
    tk0 = torch.tensor(k, dtype=torch.float64).requires_grad_(grad)
    tv0 = torch.tensor(v, dtype=torch.float64).requires_grad_(grad)
    tk = tk0.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = tv0.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    add = torch.where(torch.tensor(mask_bool), 0.0, float("-inf")).to(torch.float64)
    add = add.expand(q.shape[0], q.shape[2], q.shape[1], k.shape[1]).clone()
    tb = None
    if bias is not None:
        tb = torch.tensor(bias, dtype=torch.float64).requires_grad_(grad)
        add = add + tb
    ts = None
    if sink is not None:
        B, H, S, _ = add.shape
        ts = torch.tensor(sink, dtype=torch.float64).requires_grad_(grad)
        tk = torch.cat([tk, torch.zeros(B, H, 1, tk.shape[3], dtype=torch.float64)], dim=2)
        tv = torch.cat([tv, torch.zeros(B, H, 1, tv.shape[3], dtype=torch.float64)], dim=2)
        add = torch.cat([add, ts.view(1, H, 1, 1).expand(B, H, S, 1)], dim=3)
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=add, scale=scale)
    out = out.permute(0, 2, 1, 3)
    if not grad:
        return out.detach().numpy()
    out.backward(torch.tensor(do, dtype=torch.float64))
    return (out.detach().numpy(), tq.grad.permute(0, 2, 1, 3).numpy(), tk0.grad.numpy(), tv0.grad.numpy(),
            None if tb is None else tb.grad.numpy(), None if ts is None else ts.grad.numpy())


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


MASKS = [
    dict(causal=False, window=0, seg=False),
    dict(causal=True, window=0, seg=False),
    dict(causal=True, window=7, seg=False),
    dict(causal=False, window=5, seg=False),
    dict(causal=True, window=0, seg=True),
    dict(causal=True, window=9, seg=True),
]


@pytest.mark.parametrize("m", MASKS, ids=lambda m: "c{causal}_w{window}_s{seg}".format(**m))
@pytest.mark.parametrize("with_bias", [False, True])
def test_uncapped_equals_sdpa_forward_and_backward(m, with_bias):
    q, k, v, do, rng = _inputs()
    B, S, Hq = q.shape[0], q.shape[1], q.shape[2]
    seg = None
    if m["seg"]:
        seg = np.array([[0] * 5 + [1] * 20 + [2] * 12, [0] * 30 + [1] * 7])
    bias = rng.standard_normal((B, Hq, S, S)) if with_bias else None
    mask = _mask(S, m["causal"], m["window"], seg)
    ref = _sdpa(q, k, v, mask, bias=bias, grad=True, do=do)
    kw = dict(causal=m["causal"], window=m["window"], segment_ids=seg, bias=bias, softcap=0.0)
    out, lse = attention_forward(q, k, v, **kw)
    assert _rel(out, ref[0]) < 1e-12
    dq, dk, dv, dbias, _ = attention_backward(q, k, v, do, **kw)
    assert _rel(dq, ref[1]) < 1e-12
    assert _rel(dk, ref[2]) < 1e-12
    assert _rel(dv, ref[3]) < 1e-12
    if with_bias:
        assert _rel(dbias, ref[4]) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_sink_equals_sdpa_with_one_extra_zero_key(causal):
    q, k, v, do, rng = _inputs(seed=3)
    S, Hq = q.shape[1], q.shape[2]
    sink = rng.standard_normal(Hq) * 5
    mask = _mask(S, causal, 0, None)
    ref = _sdpa(q, k, v, mask, sink=sink, grad=True, do=do)
    out, lse = attention_forward(q, k, v, causal=causal, sink=sink)
    assert _rel(out, ref[0]) < 1e-12
    dq, dk, dv, _, dsink = attention_backward(q, k, v, do, causal=causal, sink=sink)
    for a, b in zip((dq, dk, dv, dsink), (ref[1], ref[2], ref[3], ref[5])):
        assert _rel(a, b) < 1e-11


def test_lse_matches_logsumexp_of_sdpa_scores():
    """lse is the natural log of the softmax normaliser, sink included."""
    q, k, v, do, rng = _inputs(B=1, S=20, Hq=2, Hkv=1, D=8, seed=5)
    sink = np.array([1.5, -2.0])
    _, lse = attention_forward(q, k, v, causal=True, sink=sink)
    scores = np.einsum("bihd,bjd->bhij", q, k[:, :, 0]) / np.sqrt(8)
    scores = np.where(np.tril(np.ones((20, 20), dtype=bool)), scores, -np.inf)
    full = np.concatenate([scores, np.broadcast_to(sink.reshape(1, 2, 1, 1), (1, 2, 20, 1))], axis=3)
    ref = torch.logsumexp(torch.tensor(full), dim=-1).numpy()
    assert np.max(np.abs(lse - ref)) < 1e-12


def test_custom_scale_is_used():
    q, k, v, do, rng = _inputs(B=1, S=16, Hq=2, Hkv=2, D=8)
    mask = _mask(16, True, 0, None)
    ref = _sdpa(q, k, v, mask, scale=0.3)
    out, _ = attention_forward(q, k, v, causal=True, scale=0.3)
    assert _rel(out, ref) < 1e-12


# ---- the two packed variants of the tokamax PR description: k_start and a dense boolean mask

def _kstart_loop_mask(S, causal, k_start):
    """Visibility from k_start written with loops: key j visible to query i iff j >= k_start[i]."""
    B = k_start.shape[0]
    m = np.zeros((B, 1, S, S), dtype=bool)
    for b in range(B):
        for i in range(S):
            for j in range(S):
                m[b, 0, i, j] = (j >= k_start[b, i]) and (not causal or j <= i)
    return m


def test_k_start_equals_sdpa_with_its_loop_mask():
    q, k, v, do, rng = _inputs()
    S = q.shape[1]
    k_start = np.sort(rng.integers(0, S, size=(2, S)), axis=1)      # non-decreasing, one row per batch
    got = attention_backward(q, k, v, do, causal=True, k_start=k_start)
    out, _ = attention_forward(q, k, v, causal=True, k_start=k_start)
    ref = _sdpa(q, k, v, _kstart_loop_mask(S, True, k_start), grad=True, do=do)
    # rows with no visible key are NaN in SDPA; compare the rows that see something
    ok = np.array([[k_start[b, i] <= i for i in range(S)] for b in range(2)])
    for b in range(2):
        r = ok[b]
        assert _rel(out[b, r], ref[0][b, r]) < 1e-12
        assert _rel(got[0][b, r], ref[1][b, r]) < 1e-12
    assert _rel(got[1], ref[2]) < 1e-12 and _rel(got[2], ref[3]) < 1e-12


def test_dense_mask_equals_sdpa_with_the_same_boolean_mask():
    q, k, v, do, rng = _inputs(S=29)
    S = q.shape[1]
    dense = rng.random((2, S, S)) < 0.6
    dense[:, np.arange(S), np.arange(S)] = True          # every row sees at least its own key
    got = attention_backward(q, k, v, do, mask=dense)
    out, _ = attention_forward(q, k, v, mask=dense)
    ref = _sdpa(q, k, v, dense[:, None], grad=True, do=do)
    assert _rel(out, ref[0]) < 1e-12
    for a, b in zip(got[:3], ref[1:4]):
        assert _rel(a, b) < 1e-12


def _packings(S, rng, n=4):
    """One packing (segment starts per row) written three ways: ids, k_start, dense."""
    B = 2
    seg = np.zeros((B, S), dtype=np.int64)
    for b in range(B):
        for c in np.sort(rng.choice(np.arange(1, S), n - 1, replace=False)):
            seg[b, c:] += 1
    # k_start: the first token of each token's segment, found by scanning back
    k_start = np.zeros((B, S), dtype=np.int64)
    for b in range(B):
        for i in range(S):
            x = i
            while x > 0 and seg[b, x - 1] == seg[b, i]:
                x -= 1
            k_start[b, i] = x
    dense = seg[:, :, None] == seg[:, None, :]
    return seg, k_start, dense


@pytest.mark.parametrize("softcap", [0.0, 5.0])
def test_segment_ids_k_start_and_dense_mask_agree_to_every_digit(softcap):
    """Causal packing as segment ids, as k_start and as a dense mask: the same outputs
    and gradients, bit for bit (the PR description's 'agree to every digit')."""
    q, k, v, do, rng = _inputs(S=41, seed=3)
    seg, k_start, dense = _packings(41, rng)
    kw = dict(causal=True, softcap=softcap, sink=rng.standard_normal(6))
    a = attention_forward(q, k, v, segment_ids=seg, **kw) + attention_backward(q, k, v, do, segment_ids=seg, **kw)
    b = attention_forward(q, k, v, k_start=k_start, **kw) + attention_backward(q, k, v, do, k_start=k_start, **kw)
    c = attention_forward(q, k, v, mask=dense, **kw) + attention_backward(q, k, v, do, mask=dense, **kw)
    for x, y, z in zip(a, b, c):
        if x is None:
            continue
        assert np.array_equal(x, y) and np.array_equal(x, z)
