"""GPU parity against the fp64 oracle at sizes that span several tiles with ragged tails.

Every case compares out, lse, dq, dk, dv (and dbias, dsink when present)
element by element with the oracle run on the same (bf16- or fp16-rounded)
inputs; the bar is the normwise error max|x - ref| / max|ref| <= 1e-5 (fp32
path), 1e-2 (bf16 path) or 2e-3 (fp16 path, derived in the harness).
"""
import numpy as np
import pytest

from harness import TOL, as_dense_mask, as_k_start, case, compare, rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _check(c, thd=False, backward=True, dq_mode="auto", residual=True, per_head=True, layout="bshd"):
    """Every tensor, and (per_head) every (batch row, head) slice of it, must meet the bar."""
    print(f"case: dtype={c['dtype']} q={c['q'].shape} k={c['k'].shape} causal={c['causal']} window={c['window']} "
          f"cap={c['softcap']} sink={c['sink_mode']} bias={c['bias'] is not None} "
          f"seg={c['segment_ids'] is not None} thd={thd} dq_mode={dq_mode} residual={residual} layout={layout}",
          flush=True)
    gpu = run_gpu(c, backward=backward, thd=thd, dq_mode=dq_mode, residual=residual, layout=layout)
    ref = run_oracle(c, backward=backward)
    errs = compare(gpu, ref, c["dtype"], per_head=per_head)
    whole = {k: v for k, v in errs.items() if "[" not in k}
    worst = max((v, k) for k, v in errs.items() if "[" in k) if len(errs) > len(whole) else None
    print("errors:", {k: f"{v:.2e}" for k, v in whole.items()},
          "" if worst is None else f"worst head slice {worst[1]} {worst[0]:.2e}", flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[c["dtype"]]}
    assert not bad, f"over tolerance {TOL[c['dtype']]}: {bad}"
    return whole


@pytest.mark.parametrize("dtype", ["bf16", "fp32", "fp16"])
@pytest.mark.parametrize("D", [64, 128, 256, 512])
def test_causal_gqa_cap(dtype, D):
    _check(case(dtype=dtype, D=D, B=2, S=200, Hq=4, Hkv=2, softcap=30.0, q_scale=4.0))


FEATURES = {
    "window": dict(window=37),
    "segments": dict(segments=[[45, 70, 190], [128]]),
    "bias": dict(bias=True, softcap=50.0),
    "sink_learnable": dict(sink_mode="learnable"),
    "sink_off_by_one": dict(sink_mode="off_by_one"),
    "no_causal": dict(causal=False),
    "no_cap": dict(softcap=0.0),
    "bias_and_sink": dict(bias=True, sink_mode="learnable", softcap=20.0),
    "gqa_packing_window": dict(Hq=6, Hkv=2, segments=[[13, 100], [77, 78, 150]], window=50),
    "everything": dict(Hq=8, Hkv=2, segments=[[60, 61, 131]], window=40, bias=True, sink_mode="learnable"),
    "noncausal_window_segments": dict(causal=False, window=29, segments=[[99]]),
    "mqa": dict(Hq=4, Hkv=1),
}


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("bf16", 256), ("fp32", 64),
                                     ("fp32", 256), ("bf16", 512), ("fp32", 512), ("fp16", 64), ("fp16", 128),
                                     ("fp16", 256), ("fp16", 512)])
@pytest.mark.parametrize("feat", list(FEATURES))
def test_feature_matrix(dtype, D, feat):
    kw = dict(dtype=dtype, D=D, B=2, S=203, Hq=4, Hkv=2)
    kw.update(FEATURES[feat])
    _check(case(**kw))


# The bf16 fast kernels take a bias only when Sk is a multiple of 8 (bias rows are read 16
# bytes at a time), which S = 203 above is not: these cases run them, including the dk/dv
# kernel's bias / dbias tiles and the dbias zeros it writes outside its visible query tiles.
BIAS_FAST = {
    "causal": dict(),
    "window": dict(window=37),
    "segments": dict(segments=[[45, 70, 190], [128]]),
    "no_causal": dict(causal=False),
    "no_causal_window": dict(causal=False, window=29),
    "sink_gqa_packing": dict(Hq=6, Hkv=2, segments=[[13, 100], [77, 78, 150]], window=50, sink_mode="learnable"),
}


@pytest.mark.parametrize("dtype,D,dq_mode", [("bf16", 64, "auto"), ("bf16", 64, "du_blocks"), ("bf16", 128, "auto"),
                                             ("bf16", 256, "auto"), ("fp16", 128, "auto"), ("fp16", 64, "du_blocks")])
@pytest.mark.parametrize("feat", list(BIAS_FAST))
def test_bias_on_the_fast_path(dtype, D, dq_mode, feat):
    kw = dict(dtype=dtype, D=D, B=2, S=200, Hq=4, Hkv=2, bias=True, softcap=50.0)
    kw.update(BIAS_FAST[feat])
    _check(case(**kw), dq_mode=dq_mode)


# dq_mode "auto" takes the dU hand-off at D >= 128 and recomputes at D = 64;
# each D also runs the other way here (D = 256 and 512 recompute through the
# generic dq kernel)
OTHER_DQ_MODE = {64: "du_blocks", 128: "recompute", 256: "recompute", 512: "recompute"}


@pytest.mark.parametrize("D", [128, 64, 256, 512])
@pytest.mark.parametrize("feat", list(FEATURES))
def test_feature_matrix_other_dq_mode(D, feat):
    kw = dict(dtype="bf16", D=D, B=2, S=203, Hq=4, Hkv=2)
    kw.update(FEATURES[feat])
    mode = OTHER_DQ_MODE[D]
    if mode == "du_blocks" and kw.get("bias"):
        pytest.skip("the dU hand-off needs Sk % 8 == 0 with a bias (S = 203 here); see the fast-path bias tests")
    _check(case(**kw), dq_mode=mode)


# fp32: the generic dk/dv kernel writes fp32 dU blocks that the generic dq kernel reads (auto at
# D >= 128, or with dropout), else dq recomputes; both modes at every D and feature
FP32_DQ_FEATURES = dict(FEATURES, dropout=dict(dropout_p=0.2, sink_mode="learnable"))


@pytest.mark.parametrize("dq_mode", ["du_blocks", "recompute"])
@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("feat", list(FP32_DQ_FEATURES))
def test_fp32_both_dq_modes(D, feat, dq_mode):
    kw = dict(dtype="fp32", D=D, B=2, S=203, Hq=4, Hkv=2)
    kw.update(FP32_DQ_FEATURES[feat])
    _check(case(**kw), dq_mode=dq_mode)


@pytest.mark.parametrize("D", [64, 128, 256, 512])
def test_without_the_output_residual(D):
    """bf16 without out_lo: delta comes from the bf16 output alone (the
    pre-pass's other branch); a case where that rounding stays small."""
    _check(case(dtype="bf16", D=D, B=2, S=203, Hq=4, Hkv=2, sink_mode="learnable"), residual=False)


@pytest.mark.parametrize("D", [64, 128, 256, 512])
def test_learnable_sink_above_the_cap(D):
    """Sink logits above the cap: the forward's fixed reference maximum (the
    cap) moves to the sink in the epilogue."""
    c = case(dtype="bf16", D=D, B=2, S=203, Hq=4, Hkv=2, softcap=30.0, sink_mode="learnable")
    c["sink"] = np.array([45.0, -3.0, 60.0, 29.5], dtype=np.float32)
    _check(c)


# Without a bias, D = 512 runs on the four-slice kernels.  A cap of 50 (2 c log2 e > 60) takes the
# running row maximum, whose per-tile extreme the slices exchange; cap 30 (the feature matrix)
# takes the fixed reference maximum.
WIDE_CAP50 = {
    "plain": dict(),
    "sink_learnable": dict(sink_mode="learnable"),
    "sink_off_by_one": dict(sink_mode="off_by_one"),
    "window_segments": dict(window=37, segments=[[45, 70, 190], [128]]),
    "dropout": dict(dropout_p=0.2, sink_mode="learnable"),
    "no_causal": dict(causal=False),
}


# D = 512 with a bias and Sk % 8 == 0 runs on the four-slice kernels too: each quarter's owner reads
# its pairs' bias and writes their dbias (S = 200 here; S = 203 above takes the generic kernels)
WIDE_BIAS = {
    "cap30": dict(bias=True, softcap=30.0),
    "cap50": dict(bias=True, softcap=50.0),
    "no_cap_sink": dict(bias=True, softcap=0.0, sink_mode="learnable"),
    "heads_bcast": dict(bias=True, softcap=50.0, bias_bcast="heads"),
    "batch_bcast": dict(bias=True, softcap=30.0, bias_bcast="batch"),
    "segments_window": dict(bias=True, softcap=50.0, segments=[[45, 70, 190], [128]], window=40),
    "dropout": dict(bias=True, softcap=30.0, dropout_p=0.2, sink_mode="learnable"),
    "no_causal": dict(bias=True, softcap=50.0, causal=False),
}


@pytest.mark.parametrize("dq_mode", ["auto", "recompute"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("feat", list(WIDE_BIAS))
def test_d512_bias_on_the_wide_kernels(dtype, feat, dq_mode):
    _check(case(dtype=dtype, D=512, B=2, S=200, Hq=4, Hkv=2, **WIDE_BIAS[feat]), dq_mode=dq_mode)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("feat", list(WIDE_CAP50))
def test_d512_running_maximum(dtype, feat):
    _check(case(dtype=dtype, D=512, B=2, S=203, Hq=4, Hkv=2, softcap=50.0, **WIDE_CAP50[feat]))


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("fp32", 64), ("bf16", 128), ("fp32", 256), ("bf16", 512),
                                     ("fp32", 512), ("fp16", 512)])
def test_cross_attention_lengths_differ(dtype, D):
    _check(case(dtype=dtype, D=D, B=1, S=77, Sk=301, causal=False, Hq=2, Hkv=1))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 128), ("bf16", 512), ("fp32", 512)])
def test_thd_varlen_matches_oracle(dtype, D):
    c = case(dtype=dtype, D=D, B=2, S=160, segments=[[7, 64, 65, 130], [100]], sink_mode="learnable")
    _check(c, thd=True)


@pytest.mark.parametrize("form", ["dropout", "k_start", "dense_mask"])
def test_thd_with_the_other_options(form):
    """THD (cu_seqlens, one flat token axis) together with dropout, a k_start that cuts a
    window into each sequence, or a dense band mask on top of the sequences."""
    c = case(dtype="bf16", D=128, B=1, S=230, segments=[[7, 64, 65, 130]], sink_mode="learnable",
             dropout_p=0.2 if form == "dropout" else 0.0)
    seg = c["segment_ids"][0]
    i = np.arange(230)
    start = np.array([np.nonzero(seg == seg[t])[0][0] for t in i])
    if form == "k_start":
        c["k_start"] = np.maximum(start, i - 40)[None].astype(np.int32)
    elif form == "dense_mask":
        c["mask"] = ((i[:, None] - i[None, :]) < 50)[None]
    _check(c, thd=True)


def test_thd_equals_segment_ids_bitwise():
    c = case(dtype="bf16", D=64, B=2, S=192, segments=[[50, 51, 120], [64, 128]])
    a = run_gpu(c)
    b = run_gpu(c, thd=True)
    for n in ("out", "dq", "dk", "dv"):
        assert np.array_equal(a[n].reshape(b[n].shape), b[n]), n


def _ds_conditioning(c):
    """kappa = max over rows of sum_j P_ij |dP_ij| / max_j |dS_ij| (fp64, causal, the case's cap):
    how much an error of delta, relative to the terms it sums, grows in dS = P (dP - delta)."""
    q, k, v, do = (c[n].astype(np.float64)[0] for n in ("q", "k", "v", "dout"))
    S, Hq, D = q.shape[0], q.shape[1], q.shape[2]
    G = Hq // k.shape[1]
    kap = 1.0
    for h in range(Hq):
        u = q[:, h] @ k[:, h // G].T / np.sqrt(D)
        s = c["softcap"] * np.tanh(u / c["softcap"])
        s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
        P = np.exp(s - s.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        dP = do[:, h] @ v[:, h // G].T
        dS = P * (dP - (P * dP).sum(1, keepdims=True))
        for i in range(S):
            if np.abs(dS[i]).max() > 0:
                kap = max(kap, float((P[i] * np.abs(dP[i])).sum() / np.abs(dS[i]).max()))
    return kap


@pytest.mark.parametrize("dtype,D", [("fp32", 64), ("bf16", 64), ("bf16", 128), ("fp32", 128), ("fp32", 256),
                                     ("bf16", 256), ("bf16", 512), ("fp32", 512)])
def test_single_token_and_tiny_lengths(dtype, D):
    # S = 2 (causal): the second row's probabilities can be as lopsided as 0.9999 and
    # 0.0001, so its dS (all of dq and dk) is a cancellation in dP - delta.  In bf16,
    # delta must come from the fp32 output (out + out_lo), since the rounding of a bf16
    # out alone moves it by 0.026.  In fp32 the forward's output and the backward's
    # probabilities each carry a few units of fp32 rounding, which the cancellation
    # multiplies by kappa (_ds_conditioning: about 7000 at D = 128 with this draw):
    # there the bar is 16 kappa 2^-24 (at least 1e-5), derived from that arithmetic.
    # Whole tensors only: at S = 2 a head's dq is that cancellation alone.
    for S in (1, 2, 31, 33):
        c = case(dtype=dtype, D=D, B=1, S=S, Hq=2, Hkv=1)
        if dtype == "fp32" and S == 2:
            kap = _ds_conditioning(c)
            tol = max(TOL["fp32"], 16 * kap * 2.0 ** -24)
            print(f"fp32 S=2: dS conditioning {kap:.0f}, bar {tol:.2e}", flush=True)
            gpu, ref = run_gpu(c), run_oracle(c)
            errs = {n: rel_err(gpu[n], ref[n]) for n in ("out", "lse", "dq", "dk", "dv")}
            print("errors:", {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
            assert errs["out"] <= TOL["fp32"] and errs["lse"] <= TOL["fp32"] and errs["dv"] <= TOL["fp32"], errs
            assert errs["dq"] <= tol and errs["dk"] <= tol, (errs, tol)
            continue
        _check(c, per_head=False)


def test_large_logits_cap_saturates_without_nan():
    """Pre-cap logits of several hundred, cap 30: no overflow in the 1 - t^2 factor."""
    c = case(dtype="fp32", D=64, B=1, S=150, Hq=2, Hkv=2, q_scale=60.0, softcap=30.0, window=20,
             segments=[[70]])
    errs = _check(c)
    assert all(np.isfinite(v) for v in errs.values())


@pytest.mark.parametrize("dtype,D", [("fp32", 64), ("bf16", 128), ("fp32", 256), ("bf16", 512)])
def test_fully_masked_rows_give_zero_and_minus_inf(dtype, D):
    """Non-causal window with Sq > Sk: late rows see no key."""
    c = case(dtype=dtype, D=D, B=1, S=96, Sk=32, causal=False, window=40, Hq=2, Hkv=1)
    gpu = run_gpu(c)
    ref = run_oracle(c)
    assert np.all(gpu["out"][0, 72:] == 0.0)
    assert np.all(np.isneginf(gpu["lse"][0, :, 72:]))
    errs = compare(gpu, ref, dtype)
    assert all(v <= TOL[dtype] for v in errs.values()), errs


# ---- the two other packed forms of the tokamax PR description: k_start and a dense boolean mask

PACKED = {
    "causal": dict(segments=[[45, 70, 190], [128]]),
    "window_gqa_sink": dict(Hq=6, Hkv=2, segments=[[13, 100], [77, 78, 150]], window=50, sink_mode="learnable"),
    "bias": dict(segments=[[60, 61, 131], [33]], bias=True, softcap=50.0),
}


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("bf16", 512), ("fp32", 64),
                                     ("fp32", 512), ("fp16", 64)])
@pytest.mark.parametrize("form", ["k_start", "dense_mask"])
@pytest.mark.parametrize("feat", list(PACKED))
def test_packed_forms_match_oracle(dtype, D, form, feat):
    kw = dict(dtype=dtype, D=D, B=2, S=200, Hq=4, Hkv=2)
    kw.update(PACKED[feat])
    c = case(**kw)
    _check(as_k_start(c) if form == "k_start" else as_dense_mask(c))


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("bf16", 512), ("fp32", 128)])
def test_segment_ids_k_start_and_dense_mask_agree_bitwise(dtype, D):
    """One causal packing given as segment ids, as k_start and as a dense mask: the
    kernels agree to every bit (the dense mask adds only exact zeros from pairs it removes)."""
    c = case(dtype=dtype, D=D, B=2, S=200, Hq=4, Hkv=2, segments=[[45, 70, 190], [128]], sink_mode="learnable")
    a = run_gpu(c)
    b = run_gpu(as_k_start(c))
    m = run_gpu(as_dense_mask(c))
    for n, x in a.items():
        if x is None:
            continue
        assert x.tobytes() == b[n].tobytes(), f"{n}: k_start differs from segment ids"
        assert x.tobytes() == m[n].tobytes(), f"{n}: dense mask differs from segment ids"


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64), ("bf16", 512)])
def test_random_dense_mask_and_k_start_without_causal(dtype, D):
    """A dense mask that is not a packing (random pairs, some rows empty), and a
    non-decreasing k_start without causal masking, on cross attention (Sq != Sk)."""
    rng = np.random.default_rng(5)
    c = case(dtype=dtype, D=D, B=2, S=97, Sk=150, causal=False, Hq=4, Hkv=2, sink_mode="learnable")
    m = rng.random((2, 97, 150)) < 0.3
    m[0, 10] = False                                      # a row that sees nothing: only the sink
    _check(dict(c, mask=m))
    ks = np.sort(rng.integers(0, 160, size=(2, 97)), axis=1).astype(np.int32)   # some rows past Sk: empty
    _check(dict(c, k_start=ks))


def _interval_mask(a, e, Sk):
    j = np.arange(Sk)[None, None, :]
    return (j >= a[:, :, None]) & (j < e[:, :, None])


DENSE_INTERVALS = ["monotone", "not_monotone", "mixed_rows", "causal_band_with_segments"]


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("bf16", 512), ("fp32", 64),
                                     ("fp16", 128)])
@pytest.mark.parametrize("kind", DENSE_INTERVALS)
def test_dense_masks_of_key_intervals(dtype, D, kind):
    """Dense masks whose rows are key intervals.  Where the intervals' ends do not
    decrease down the rows the library describes the mask by per-row ranges alone
    (no per-pair mask reads); otherwise, and in a batch row with a gap inside a row,
    it reads the mask pair by pair inside wider ranges.  Both against the oracle."""
    rng = np.random.default_rng(11)
    B, S, Sk = 2, 203, 203
    causal = kind == "causal_band_with_segments"
    kw = dict(dtype=dtype, D=D, B=B, S=S, Hq=4, Hkv=2, causal=causal, sink_mode="learnable")
    if causal:
        kw["segments"] = [[45, 70, 190], [128]]
    c = case(**kw)
    if kind == "monotone":
        a = np.sort(rng.integers(0, Sk, size=(B, S)), axis=1)
        e = np.maximum(a + 1, np.sort(rng.integers(0, Sk + 1, size=(B, S)), axis=1))
        m = _interval_mask(a, e, Sk)
    elif kind == "not_monotone":
        a = rng.integers(0, Sk, size=(B, S))
        e = np.minimum(a + rng.integers(1, 90, size=(B, S)), Sk)
        m = _interval_mask(a, e, Sk)
    elif kind == "mixed_rows":
        a = np.sort(rng.integers(0, Sk, size=(B, S)), axis=1)
        e = np.maximum(a + 1, np.sort(rng.integers(0, Sk + 1, size=(B, S)), axis=1))
        m = _interval_mask(a, e, Sk)
        m[1, 100, (a[1, 100] + e[1, 100]) // 2] = False   # a gap inside one row of batch row 1
        m[1, 150] = False                                   # and a row that sees nothing
    else:
        i = np.arange(S)[:, None]
        j = np.arange(Sk)[None, :]
        m = np.broadcast_to((i - j < 37) & (j <= i + 5), (B, S, Sk)).copy()   # a band, cut by causal
    _check(dict(c, mask=m))


# ---- a bias broadcast over batch rows and/or heads: dbias of the bias's own shape

@pytest.mark.parametrize("dtype,D,S", [("bf16", 64, 200), ("bf16", 128, 200), ("bf16", 256, 200),
                                       ("bf16", 512, 203), ("fp32", 128, 203), ("fp16", 64, 200)])
@pytest.mark.parametrize("bcast", ["batch", "heads", "batch_heads"])
def test_broadcast_bias(dtype, D, S, bcast):
    c = case(dtype=dtype, D=D, B=2, S=S, Hq=4, Hkv=2, bias=True, softcap=50.0, bias_bcast=bcast,
             segments=[[45, 70, 190], [128]], sink_mode="learnable")
    errs = _check(c)
    assert "dbias" in errs


# ---- SBHD layout ([S, B, H, D], the sbhd rows of the learnable-sink page's verification table)

SBHD = {
    "bf16_d64_split": (dict(dtype="bf16", D=64, B=2, S=203, Hq=8, Hkv=2, sink_mode="learnable"), "auto"),
    "bf16_d64_du": (dict(dtype="bf16", D=64, B=2, S=200, Hq=4, Hkv=2, bias=True, segments=[[45, 70], [128]]),
                    "du_blocks"),
    "bf16_d128_bias": (dict(dtype="bf16", D=128, B=3, S=200, Hq=4, Hkv=2, bias=True, softcap=50.0,
                            segments=[[45, 70, 190], [128], [5]]), "auto"),
    "bf16_d128_recompute": (dict(dtype="bf16", D=128, B=2, S=203, Hq=4, Hkv=1, window=37), "recompute"),
    "bf16_d256": (dict(dtype="bf16", D=256, B=2, S=203, Hq=4, Hkv=2, sink_mode="learnable"), "auto"),
    "bf16_d512": (dict(dtype="bf16", D=512, B=2, S=150, Hq=2, Hkv=1, sink_mode="learnable"), "auto"),
    "bf16_d512_bias": (dict(dtype="bf16", D=512, B=2, S=150, Hq=2, Hkv=1, bias=True), "auto"),
    "fp32_d128": (dict(dtype="fp32", D=128, B=2, S=203, Hq=4, Hkv=2, sink_mode="learnable", window=50), "auto"),
    "fp16_d64": (dict(dtype="fp16", D=64, B=2, S=203, Hq=4, Hkv=2, causal=False), "auto"),
}


@pytest.mark.parametrize("name", list(SBHD))
def test_sbhd_layout_matches_oracle_and_bshd(name):
    kw, mode = SBHD[name]
    c = case(**kw)
    _check(c, dq_mode=mode, layout="sbhd")
    a = run_gpu(c, dq_mode=mode)
    b = run_gpu(c, dq_mode=mode, layout="sbhd")
    for n, x in a.items():
        if x is not None:
            assert x.tobytes() == b[n].tobytes(), f"{name}: {n} differs between BSHD and SBHD"


# ---- dropout inside the kernels: the same Philox4x32-10 keep decisions as the oracle's

DROPOUT = {
    "causal": dict(),
    "sink_bias": dict(sink_mode="learnable", bias=True, softcap=50.0),
    "segments_window": dict(segments=[[45, 70, 190], [128]], window=60, Hq=6, Hkv=2),
    "no_causal_cross": dict(causal=False, Sk=150, softcap=0.0),
    "sink_bias_fast": dict(S=200, sink_mode="learnable", bias=True, softcap=30.0),   # Sk % 8 == 0: fast kernels
}


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("bf16", 512), ("fp16", 128),
                                     ("fp16", 256), ("fp32", 64), ("fp32", 256)])
@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("feat", list(DROPOUT))
def test_dropout_matches_oracle(dtype, D, p, feat):
    kw = dict(dtype=dtype, D=D, B=2, S=203, Hq=4, Hkv=2, dropout_p=p)
    kw.update(DROPOUT[feat])
    _check(case(**kw))


@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("dq_mode", ["du_blocks", "recompute"])
def test_dropout_on_the_fast_dkdv_kernel_both_dq_modes(D, dq_mode):
    """The fast dk/dv kernel with dropout hands dq either its dU blocks or leaves dq to the
    recomputing (generic) kernel; both against the oracle, over several query tiles and a
    query-head split (B * Hkv * key blocks < 1024)."""
    c = case(dtype="bf16", D=D, B=2, S=333, Hq=8, Hkv=2, softcap=30.0, sink_mode="learnable", dropout_p=0.2)
    _check(c, dq_mode=dq_mode)
