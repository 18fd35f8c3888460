"""fp64 CPU oracle: attention with a tanh logit soft-cap and a softmax sink.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the bench's ``cpu_baseline`` leg may import or run this module.  It shares
no code with the HIP path (no kernels, headers, tables or helpers) and
never imports it.

What it computes is the plain materialised definition, written out in NumPy
float64 for one (batch row, KV head) group at a time and a block of query
rows at a time; nothing is tiled over keys and there is no online softmax, so
each line can be checked against the sources by eye:

* "Thread tanh logit softcapping through FlashAttention (FA2, opt-in FA3)",
  intro and "What changed": logits are soft-capped as ``cap*tanh(x/cap)``;
  ``softcap = 0`` is the default and leaves attention unchanged.
* "Support logits soft-capping in the Pallas-Triton attention VJP", PR
  description: the cap is applied after the bias add and before masking;
  the backward multiplies ``ds`` by ``1 - tanh(u/c)^2``, that factor is
  taken before masking while the logits are finite, and dk and dbias are
  both gradients with respect to the pre-cap logits ``u``.
* The MaxText commit message quoted on that page: packed rows attend only
  inside their own segment (causal inside the segment), sliding-window
  masking, native GQA/MQA without repeating K/V.
* "learnable softmax sink with context-parallel p2p" (TransformerEngine
  PR #3551), "What changed": the sink is one more softmax column per query
  head, counted exactly once per query row; its gradient is a sum over the
  query rows.  Off-by-one softmax is that column with its logit fixed at 0.
* The bias is added after the ``1/sqrt(D)`` scale (``post_scale_bias`` in
  the Greptile review "Offset Corrupts Bias Gradient Shape" on that page).
* The same review: the bias gradient has the bias's own shape, so a bias
  broadcast over batch rows or heads ([1 or B, 1 or Hq, Sq, Sk]) gets the
  full gradient summed over the broadcast dimensions.
* Dropout inside the fused kernel: the tokamax PR description keeps
  ``dropout_mask`` out of its cases and the MaxText commit quoted there
  rejects packing with dropout where the fallback kernels have none; the
  learnable-sink page ("What changed") carries the rng state among the
  forward's auxiliary outputs.  Read here as the usual attention dropout:
  after the softmax, each probability is kept with probability 1 - p' and
  scaled by 1/(1 - p'); lse is that of the softmax before dropout.  The keep
  decisions compare 16-bit draws of a counter-based generator
  (``oracle/philox.py``), keyed by the caller's seed and offset, with a
  threshold, so p' is p rounded down to a multiple of 2^-16 (the pages fix
  no generator or precision for these draws).
* "Support logits soft-capping in the Pallas-Triton attention VJP", PR
  description: besides segment ids, a packed batch can be given as
  ``k_start`` (per query, the first key it may see) or as a dense boolean
  mask; both only remove pairs, on top of the other masks.

Readings taken where the pages are silent (each one also listed in the
design notes):  scale ``tau = 1/sqrt(D)`` unless given; the sink logit is
neither scaled nor capped; one sink logit per *query* head; a causal
sliding window of ``W`` keeps ``0 <= i-j < W`` (``|i-j| < W`` without
causal); segment visibility is equality of segment ids; ``k_start[i]`` is
the first key query ``i`` may see (keys ``j >= k_start[i]``) and a dense
mask entry True means visible, both intersected with the other masks; a row
that sees no key and has no sink gets ``out = 0``, ``lse = -inf`` and zero
gradients.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

_f64 = np.float64


def visibility(Sq: int, Sk: int, causal: bool, window: int,
               seg_q: Optional[np.ndarray] = None, seg_k: Optional[np.ndarray] = None,
               rows: Optional[slice] = None, k_start: Optional[np.ndarray] = None,
               dense: Optional[np.ndarray] = None) -> np.ndarray:
    """Boolean [rows, Sk]: may query ``i`` see key ``j``?

    visible = same segment  and  (not causal or j <= i)  and
              (W <= 0 or (0 <= i-j < W if causal else |i-j| < W))  and
              (no k_start or j >= k_start[i])  and  (no dense mask or dense[i, j]).
    """
    rows = rows if rows is not None else slice(0, Sq)
    i = np.arange(Sq)[rows][:, None]
    j = np.arange(Sk)[None, :]
    vis = np.ones((i.shape[0], Sk), dtype=bool)
    if causal:
        if Sq != Sk:
            raise ValueError("causal masking needs Sq == Sk")
        vis &= j <= i
    if window > 0:
        vis &= (i - j < window) if causal else (np.abs(i - j) < window)
    if seg_q is not None:
        vis &= seg_q[rows][:, None] == seg_k[None, :]
    if k_start is not None:
        vis &= j >= np.asarray(k_start)[rows][:, None]
    if dense is not None:
        vis &= np.asarray(dense, dtype=bool)[rows]
    return vis


def _logits(qb, k, scale, bias_rows, softcap):
    """u = tau*q.k + bias; s = cap(u); f = ds/du (all fp64, unmasked)."""
    u = scale * (qb @ k.T)
    if bias_rows is not None:
        u = u + bias_rows
    if softcap > 0.0:
        t = np.tanh(u / softcap)
        return softcap * t, 1.0 - t * t
    return u, None


def _softmax_rows(s, vis, sink_logit):
    """Masked row softmax with an optional sink column (counted once).

    Returns P (zero where masked), the sink probability p, and lse
    (natural log of the normaliser, sink included).
    """
    s_m = np.where(vis, s, -np.inf)
    m = s_m.max(axis=1)
    if sink_logit is not None:
        m = np.maximum(m, sink_logit)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.where(vis, np.exp(s_m - m_safe[:, None]), 0.0)
    z = e.sum(axis=1)
    e_sink = None
    if sink_logit is not None:
        e_sink = np.exp(sink_logit - m_safe)
        z = z + e_sink
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.where(z > 0, 1.0 / z, 0.0)
        lse = np.where(z > 0, m_safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    P = e * inv[:, None]
    p_sink = e_sink * inv if e_sink is not None else None
    return P, p_sink, lse


def group_forward(q, k, v, *, scale=None, softcap=0.0, causal=False, window=0,
                  bias=None, seg=None, sink=None, k_start=None, dense=None, dropout=None, row_block=1024):
    """Forward pass of one (batch row, KV head) group.

    q [Sq,G,D]; k, v [Sk,D]; bias [G,Sq,Sk] or None; seg [S] segment ids or
    None; sink [G] sink logits (off-by-one: zeros) or None; k_start [Sq] or
    None; dense [Sq,Sk] boolean mask or None; dropout (p, keep) with
    keep(g, rows) the boolean keep decisions [rows, Sk] of head g, or None.
    Returns out [Sq,G,D] and lse [G,Sq] in fp64.
    """
    q, k, v = (np.asarray(x, dtype=_f64) for x in (q, k, v))
    Sq, G, D = q.shape
    Sk = k.shape[0]
    scale = 1.0 / math.sqrt(D) if not scale else float(scale)
    out = np.zeros((Sq, G, v.shape[1]), dtype=_f64)
    lse = np.zeros((G, Sq), dtype=_f64)
    for r0 in range(0, Sq, row_block):
        rows = slice(r0, min(Sq, r0 + row_block))
        vis = visibility(Sq, Sk, causal, window, seg, seg, rows, k_start, dense)
        for g in range(G):
            brow = None if bias is None else np.asarray(bias[g, rows], dtype=_f64)
            s, _ = _logits(q[rows, g], k, scale, brow, softcap)
            P, _, l = _softmax_rows(s, vis, None if sink is None else float(sink[g]))
            if dropout is not None:
                P = P * dropout[1](g, rows) / (1.0 - dropout[0])
            out[rows, g] = P @ v
            lse[g, rows] = l
    return out, lse


def group_backward(q, k, v, dout, *, scale=None, softcap=0.0, causal=False, window=0,
                   bias=None, seg=None, sink=None, k_start=None, dense=None, dropout=None, want_dbias=None,
                   row_block=1024):
    """Backward pass of one (batch row, KV head) group, by recomputation.

    Returns dq [Sq,G,D], dk [Sk,D], dv [Sk,D], dbias [G,Sq,Sk] (or None) and
    dsink [G] (or None) -- this group's share of the sink gradient, i.e. the
    sum over its query rows only.
    """
    q, k, v, dout = (np.asarray(x, dtype=_f64) for x in (q, k, v, dout))
    Sq, G, D = q.shape
    Sk = k.shape[0]
    scale = 1.0 / math.sqrt(D) if not scale else float(scale)
    want_dbias = (bias is not None) if want_dbias is None else want_dbias
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dbias = np.zeros((G, Sq, Sk), dtype=_f64) if want_dbias else None
    dsink = np.zeros(G, dtype=_f64) if sink is not None else None
    for r0 in range(0, Sq, row_block):
        rows = slice(r0, min(Sq, r0 + row_block))
        vis = visibility(Sq, Sk, causal, window, seg, seg, rows, k_start, dense)
        for g in range(G):
            brow = None if bias is None else np.asarray(bias[g, rows], dtype=_f64)
            s, f = _logits(q[rows, g], k, scale, brow, softcap)
            P, p_sink, _ = _softmax_rows(s, vis, None if sink is None else float(sink[g]))
            do = dout[rows, g]
            dP = do @ v.T                              # dL/dP
            Pd = P                                     # the probabilities that multiply V
            if dropout is not None:
                kd = dropout[1](g, rows) / (1.0 - dropout[0])
                Pd = P * kd
                dP = dP * kd                           # through the kept, rescaled probabilities
            delta = (P * dP).sum(axis=1)               # sum_j P_ij dP_ij (sink column has no value)
            dS = P * (dP - delta[:, None])             # softmax Jacobian, sink column included
            dU = dS * f if f is not None else dS       # chain through the cap: 1 - tanh(u/c)^2
            if dbias is not None:
                dbias[g, rows] = dU
            dq[rows, g] = scale * (dU @ k)
            dk += scale * (dU.T @ q[rows, g])
            dv += Pd.T @ do
            if dsink is not None:
                dsink[g] -= float((p_sink * delta).sum())   # dL/dsigma = -sum_i p_i delta_i
    return dq, dk, dv, dbias, dsink


def segments_from_cu_seqlens(cu_seqlens, total: int) -> np.ndarray:
    """cu_seqlens [n+1] (cumulative lengths) -> segment id per token [total]."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to the token count")
    seg = np.zeros(total, dtype=np.int64)
    for n in range(len(cu) - 1):
        seg[cu[n]:cu[n + 1]] = n
    return seg


def _prepare(q, k, v, bias, segment_ids, cu_seqlens, k_start=None, mask=None):
    if cu_seqlens is not None:
        if segment_ids is not None:
            raise ValueError("give segment_ids or cu_seqlens, not both")
        T = q.shape[0]
        segment_ids = segments_from_cu_seqlens(cu_seqlens, T)[None, :]
        q, k, v = q[None], k[None], v[None]
        if bias is not None:
            bias = bias[None]
        k_start = None if k_start is None else np.asarray(k_start)[None]
        mask = None if mask is None else np.asarray(mask)[None]
        return q, k, v, bias, segment_ids, k_start, mask, True
    return q, k, v, bias, segment_ids, k_start, mask, False


def _dropout(p, seed, offset, b, hq0, Hq, Sk):
    """(drop probability, keep) for the group whose first query head is hq0, or None without
    dropout.  The drop probability is p rounded down to a multiple of 2^-16 (the keep decisions
    compare 16-bit draws), so that 1 / (1 - it) makes the kept values' expectation exact."""
    if not p:
        return None
    from .philox import drop_probability, dropout_keep

    def keep(g, rows):
        r = np.arange(rows.start, rows.stop) if isinstance(rows, slice) else np.asarray(rows)
        return dropout_keep(b, hq0 + g, Hq, r, Sk, p, seed, offset)
    return (drop_probability(p), keep)


def _groups(B, Hkv, groups):
    return [(b, h) for b in range(B) for h in range(Hkv)] if groups is None else list(groups)


def attention_forward(q, k, v, *, softcap=0.0, causal=False, window=0, scale=None,
                      bias=None, segment_ids=None, cu_seqlens=None, sink=None, k_start=None,
                      mask=None, dropout_p=0.0, dropout_seed=0, dropout_offset=0, groups=None):
    """Whole forward in BSHD layout (THD when ``cu_seqlens`` is given).

    q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] (THD: [T,H,D]); bias [B,Hq,Sq,Sk];
    segment_ids [B,S]; sink [Hq] (zeros for off-by-one); k_start [B,Sq]
    (THD: [T]); mask [B,Sq,Sk] boolean, True = visible (THD: [T,T]).
    ``groups`` limits the work to a list of (b, kv_head) pairs; other entries
    stay NaN.  Returns out (as q's shape) and lse [B,Hq,Sq] ([Hq,T] for
    THD), fp64.
    """
    q, k, v, bias, seg, k_start, mask, thd = _prepare(q, k, v, bias, segment_ids, cu_seqlens, k_start, mask)
    B, Sq, Hq, D = q.shape
    if bias is not None:
        bias = np.broadcast_to(bias, (B, Hq, Sq, k.shape[1]))
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    out = np.full((B, Sq, Hq, v.shape[3]), np.nan)
    lse = np.full((B, Hq, Sq), np.nan)
    for b, h in _groups(B, Hkv, groups):
        hs = slice(h * G, (h + 1) * G)
        o, l = group_forward(q[b, :, hs], k[b, :, h], v[b, :, h], scale=scale, softcap=softcap,
                             causal=causal, window=window,
                             bias=None if bias is None else bias[b, hs],
                             seg=None if seg is None else seg[b],
                             sink=None if sink is None else sink[hs],
                             k_start=None if k_start is None else k_start[b],
                             dense=None if mask is None else mask[b],
                             dropout=_dropout(dropout_p, dropout_seed, dropout_offset, b, h * G, Hq, k.shape[1]))
        out[b, :, hs] = o
        lse[b, hs] = l
    if thd:
        return out[0], lse[0]
    return out, lse


def attention_backward(q, k, v, dout, *, softcap=0.0, causal=False, window=0, scale=None,
                       bias=None, segment_ids=None, cu_seqlens=None, sink=None, k_start=None,
                       mask=None, dropout_p=0.0, dropout_seed=0, dropout_offset=0, want_dbias=None, groups=None):
    """Whole backward: dq, dk, dv, dbias (or None), dsink (or None), fp64.

    dsink sums over every batch row and query row that ``groups`` covers.
    """
    thd = cu_seqlens is not None
    q, k, v, bias, seg, k_start, mask, _ = _prepare(q, k, v, bias, segment_ids, cu_seqlens, k_start, mask)
    if thd:
        dout = dout[None]
    B, Sq, Hq, D = q.shape
    bias_shape = None
    if bias is not None:
        bias_shape = np.shape(bias)
        bias = np.broadcast_to(bias, (B, Hq, Sq, k.shape[1]))
    Hkv = k.shape[2]
    G = Hq // Hkv
    want_dbias = (bias is not None) if want_dbias is None else want_dbias
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    dbias = np.full((B, Hq, Sq, k.shape[1]), np.nan) if want_dbias else None
    dsink = np.zeros(Hq) if sink is not None else None
    for b, h in _groups(B, Hkv, groups):
        hs = slice(h * G, (h + 1) * G)
        r = group_backward(q[b, :, hs], k[b, :, h], v[b, :, h], dout[b, :, hs], scale=scale,
                           softcap=softcap, causal=causal, window=window,
                           bias=None if bias is None else bias[b, hs],
                           seg=None if seg is None else seg[b],
                           sink=None if sink is None else sink[hs],
                           k_start=None if k_start is None else k_start[b],
                           dense=None if mask is None else mask[b],
                           dropout=_dropout(dropout_p, dropout_seed, dropout_offset, b, h * G, Hq, k.shape[1]),
                           want_dbias=want_dbias)
        dq[b, :, hs], dk[b, :, h], dv[b, :, h] = r[0], r[1], r[2]
        if dbias is not None:
            dbias[b, hs] = r[3]
        if dsink is not None:
            dsink[hs] += r[4]
    if dbias is not None and tuple(bias_shape) != dbias.shape:
        # the gradient of a broadcast bias: summed over the dimensions it was broadcast along
        axes = tuple(a for a in (0, 1) if bias_shape[a] == 1 and dbias.shape[a] != 1)
        dbias = dbias.sum(axis=axes, keepdims=True)
    if thd:
        return dq[0], dk[0], dv[0], (None if dbias is None else dbias[0]), dsink
    return dq, dk, dv, dbias, dsink
