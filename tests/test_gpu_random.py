"""Seeded random combinations of the options, each checked against the oracle.

The other parity tests vary one or two options at a time around a fixed case.
Here every case draws all of them at once from a fixed seed:
- dtype, D, the GQA shape, B and S (ragged: not a tile multiple);
- Sk != Sq when nothing needs them equal;
- causal and the window;
- the cap, including 0 for no cap;
- the sink;
- the bias and its broadcast;
- dropout;
- the packed form: segment ids, k_start, a dense mask, or THD; or a drawn
  k_start (a lookback of at least 4 keys, a leading stretch of queries that
  see no key, and a jump that leaves a stretch of such queries mid-sequence,
  their empty key ranges beyond them) or a random dense mask (some rows
  empty), with Sq != Sk where nothing needs them equal;
- the dQ mode and the layout.

The backward always gets the forward's residual (out_lo): without it delta
comes from the rounded output, which the header documents as less accurate
for the gradients that go through delta, and dedicated tests cover it.

This crosses paths that the per-feature tests reach only one by one, for
example the D = 512 bias kernels under dropout in SBHD with a dense mask.

Every draw is one that the library accepts:
- causal and packing need Sq == Sk;
- THD needs B == 1;
- ATTN_DQ_DU_BLOCKS with a 16-bit bias needs Sk % 8 == 0.

The bars are those of the other parity tests (harness.TOL), per tensor and per
(batch row, head) slice.  Segments are at least 4 tokens long and fp32 cases
have S >= 17.  That keeps every row's dS away from the near-total cancellation
of two-key rows, which the tiny-length test covers with its own derived bar.

Two readings of the bars follow from the arithmetic, not from the kernels:
- dsink = -sum_i p_sink,i delta_i is one sum per head whose terms can cancel to
  a small fraction of their absolute sum.  Each term carries the rounding of
  delta = <dO, O>, so the error of the sum is bounded relative to
  sum_i p_sink,i sum_d |dO_id O_id|, and that is the scale its error is divided by.
- fp16 sinks are drawn with a spread of 2 instead of 5.  A sink logit 15 above a
  row's logits leaves the keys 1e-7 of the mass, and that head's whole output
  then lies below fp16's normal range (2^-14).  There the format's own spacing
  (2^-24) is more than the bar allows.
"""
from __future__ import annotations

import numpy as np
import pytest

from harness import TOL, as_dense_mask, as_k_start, case, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

N_CASES = 240


def _segments(rng, S):
    """Segment starts (cut points) for one batch row: pieces of at least 4 tokens."""
    cuts, t = [], 0
    while True:
        t += int(rng.integers(4, max(5, S // 2)))
        if t > S - 4:
            return cuts
        cuts.append(t)


def draw(seed):
    """One case's options: (case kwargs, run kwargs, packed form, a short description)."""
    rng = np.random.default_rng(1000 + seed)
    dtype = str(rng.choice(["bf16", "fp16", "fp32"]))
    D = int(rng.choice([64, 128, 256, 512]))
    Hkv = int(rng.choice([1, 2]))
    Hq = Hkv * int(rng.choice([1, 2, 3, 4]))
    form = str(rng.choice(["none", "none", "segments", "k_start", "dense_mask", "thd", "k_start_rand",
                           "dense_rand"]))
    B = 1 if form == "thd" else int(rng.choice([1, 2]))
    S = int(rng.integers(17, 261))
    causal = bool(rng.random() < 0.6)
    window = int(rng.integers(8, 81)) if rng.random() < 0.4 else 0
    Sk = None
    if not causal and form in ("none", "k_start_rand", "dense_rand") and rng.random() < 0.5:
        Sk = int(rng.integers(17, 261))
    softcap = float(rng.choice([0.0, 20.0, 30.0, 50.0]))
    q_scale = float(rng.choice([1.0, 4.0]))
    sink_mode = str(rng.choice(["none", "off_by_one", "learnable"]))
    bias = bool(rng.random() < 0.4)
    bias_bcast = str(rng.choice(["", "batch", "heads", "batch,heads"])) if bias else ""
    dropout_p = float(rng.choice([0.1, 0.25])) if rng.random() < 0.3 else 0.0
    segments = None
    if form in ("segments", "k_start", "dense_mask", "thd"):
        segments = [_segments(rng, S) for _ in range(B)]
    kw = dict(dtype=dtype, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, causal=causal, window=window, softcap=softcap,
              q_scale=q_scale, sink_mode=sink_mode, bias=bias, segments=segments, seed=seed, Sk=Sk,
              bias_bcast=bias_bcast, dropout_p=dropout_p)

    sk = S if Sk is None else Sk
    du_ok = dtype == "fp32" or not bias or sk % 8 == 0
    modes = ["auto", "recompute"] + (["du_blocks"] if du_ok else [])
    run = dict(dq_mode=str(rng.choice(modes)), residual=True,
               layout="bshd" if form == "thd" else str(rng.choice(["bshd", "sbhd"])))
    return kw, run, form


def build(seed):
    kw, run, form = draw(seed)
    c = case(**kw)
    if c["dtype"] == "fp16" and c["sink"] is not None:   # keep fp16 outputs in the normal range
        c["sink"] = (c["sink"] * 0.4).astype(np.float32)
    if form == "k_start":
        c = as_k_start(c)
        if c["window"] == 0 and seed % 2:   # a k_start that also cuts a window into each segment
            i = np.arange(c["q"].shape[1])
            c["k_start"] = np.maximum(c["k_start"], i[None] - 30).astype(np.int32)
    elif form == "dense_mask":
        c = as_dense_mask(c)
        if seed % 2:                         # drop a band of pairs on top of the packing
            i = np.arange(c["q"].shape[1])
            c["mask"] = c["mask"] & ((i[:, None] - i[None, :]) < 45)[None]
    elif form in ("k_start_rand", "dense_rand"):
        rng = np.random.default_rng(5000 + seed)
        B, S, Sk = c["q"].shape[0], c["q"].shape[1], c["k"].shape[1]
        if form == "k_start_rand":
            # first key max(b0, i - L) before row cut, max(jump, i - L) from it: non-decreasing;
            # rows below b0, and rows cut .. jump - 1, see no key (causal)
            L = int(rng.integers(4, S + 1))
            b0 = int(rng.integers(0, S // 4 + 1))
            cut = int(rng.integers(b0, S + 1))
            jump = int(rng.integers(cut, S + 1))
            i = np.arange(S)
            ks = np.clip(np.where(i < cut, np.maximum(b0, i - L), np.maximum(jump, i - L)), 0, Sk)
            if not c["causal"]:
                ks = np.where(ks > Sk - 4, Sk, ks)    # at least 4 keys, or none
            c["k_start"] = np.broadcast_to(ks, (B, S)).astype(np.int32).copy()
        else:
            mask = rng.random((B, S, Sk)) < 0.7
            mask[:, rng.choice(S, size=3, replace=False)] = False
            c["mask"] = mask
    return c, run, form


def describe(seed):
    kw, run, form = draw(seed)
    keep = ("dtype", "B", "S", "Sk", "Hq", "Hkv", "D", "causal", "window", "softcap", "q_scale", "sink_mode",
            "bias", "bias_bcast", "dropout_p")
    return " ".join(f"{k}={kw[k]}" for k in keep) + f" form={form} " + " ".join(f"{k}={v}" for k, v in run.items())


def dsink_scale(c, ref):
    """Per query head: sum over batch rows and queries of p_sink * sum_d |dO O|, the absolute sum
    of dsink's terms with delta's own terms taken absolutely (fp64, from the oracle)."""
    absd = np.abs(ref["out"] * c["dout"].astype(np.float64)).sum(-1)      # [B, S, Hq]
    p_sink = np.exp(c["sink"].astype(np.float64)[None, :, None] - ref["lse"])  # [B, Hq, S]
    return (p_sink * absd.transpose(0, 2, 1)).sum(axis=(0, 2))


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_combination_matches_oracle(seed):
    print(f"seed {seed}: {describe(seed)}", flush=True)
    c, run, form = build(seed)
    gpu = run_gpu(c, thd=form == "thd", **run)
    ref = run_oracle(c)
    errs = compare(gpu, ref, c["dtype"], per_head=True)
    if ref.get("dsink") is not None:
        scale = dsink_scale(c, ref).max()
        d = float(np.abs(gpu["dsink"] - ref["dsink"]).max())
        errs["dsink"] = d / scale if scale > 0 else d    # no query sees a key: dsink is exactly 0
    whole = {k: f"{v:.2e}" for k, v in errs.items() if "[" not in k}
    print("errors:", whole, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[c["dtype"]]}
    assert not bad, f"over tolerance {TOL[c['dtype']]}: {bad}"
