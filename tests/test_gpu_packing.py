"""Leakage across packed segments on the GPU (the packing checks of the MaxText commit quoted on
"Support logits soft-capping in the Pallas-Triton attention VJP": a packed batch against its
segments run alone, with errors either side of a tile-unaligned boundary).

* Perturbing every input row of one segment (q, k, v, dout) leaves every output of the other
  segments bitwise unchanged: out, lse, dq, dk, dv, and dbias everywhere outside the segment's
  own block.  A masked pair contributes an exact zero, so nothing of the perturbed segment can
  reach the others.
* The packed batch against each segment run alone as a batch row of its own: the packed run's
  rows of the segment, and the GPU run of the segment alone, each against the oracle on the
  segment alone, to the dtype's bar, with the error also taken over the rows on either side of
  every boundary.
"""
import numpy as np
import pytest

from harness import TOL, case, rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

CUTS = [[45, 70, 190], [128]]          # tile-unaligned boundaries; S = 200


def _segments(row_cuts, S):
    edges = [0] + list(row_cuts) + [S]
    return [(a, e) for a, e in zip(edges[:-1], edges[1:]) if e > a]


VARIANTS = {
    "sink": dict(sink_mode="learnable"),
    "bias_window": dict(bias=True, softcap=50.0, window=40),
    "dropout": dict(dropout_p=0.2, sink_mode="learnable"),
}


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("bf16", 512), ("fp32", 128),
                                     ("fp16", 128)])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_perturbing_one_segment_leaves_the_others_bit_identical(dtype, D, variant):
    c = case(dtype=dtype, D=D, B=2, S=200, Hq=4, Hkv=2, segments=CUTS, **VARIANTS[variant])
    b, a, e = 0, 45, 70                  # the second segment of batch row 0
    rng = np.random.default_rng(99)
    c2 = dict(c)
    for n, scale in (("q", 4.0), ("k", 1.0), ("v", 1.0), ("dout", 1.0)):
        x = c[n].copy()
        x[b, a:e] = (rng.standard_normal(x[b, a:e].shape) * scale).astype(np.float32)
        c2[n] = x
    print(f"perturb segment [{a}, {e}) of batch row {b}: dtype={dtype} D={D} {variant}", flush=True)
    r1, r2 = run_gpu(c), run_gpu(c2)
    keep_t = np.ones(200, dtype=bool)
    keep_t[a:e] = False
    for n in ("out", "dq", "dk", "dv"):
        assert np.array_equal(r1[n][1], r2[n][1]), f"{n}: batch row 1 changed"
        assert np.array_equal(r1[n][b, keep_t], r2[n][b, keep_t]), f"{n}: other segments of batch row {b} changed"
    assert np.array_equal(r1["lse"][1], r2["lse"][1]) and np.array_equal(r1["lse"][b][:, keep_t],
                                                                          r2["lse"][b][:, keep_t]), "lse changed"
    # the perturbed segment's own outputs did change (the test would pass vacuously otherwise)
    assert not np.array_equal(r1["out"][b, a:e], r2["out"][b, a:e])
    if r1["dbias"] is not None:
        d1, d2 = r1["dbias"].copy(), r2["dbias"].copy()
        d1[b, :, a:e, a:e] = 0.0
        d2[b, :, a:e, a:e] = 0.0
        assert np.array_equal(d1, d2), "dbias changed outside the perturbed segment's block"


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("bf16", 512), ("fp32", 64)])
@pytest.mark.parametrize("variant", ["sink", "bias_window"])
def test_packed_batch_matches_segments_run_alone(dtype, D, variant):
    c = case(dtype=dtype, D=D, B=2, S=200, Hq=4, Hkv=2, segments=CUTS, **VARIANTS[variant])
    packed = run_gpu(c)
    tol = TOL[dtype]
    for b in range(2):
        for a, e in _segments(CUTS[b], 200):
            alone = dict(c, segment_ids=None, q=c["q"][b:b + 1, a:e], k=c["k"][b:b + 1, a:e],
                         v=c["v"][b:b + 1, a:e], dout=c["dout"][b:b + 1, a:e],
                         bias=None if c["bias"] is None else c["bias"][b:b + 1, :, a:e, a:e])
            r = run_gpu(alone)
            ref = run_oracle(alone)
            edge = np.r_[0:min(8, e - a), max(0, e - a - 8):e - a]    # rows on either side of the boundaries
            errs = {}
            for name, got in (("packed", {n: None if packed[n] is None else packed[n][b:b + 1] for n in packed}),
                              ("alone", r)):
                sl = (lambda x: x[:, a:e]) if name == "packed" else (lambda x: x)   # noqa: E731
                errs[f"{name}.out"] = rel_err(sl(got["out"])[0], ref["out"][0])
                errs[f"{name}.lse"] = rel_err(got["lse"][0][:, a:e] if name == "packed" else got["lse"][0],
                                              ref["lse"][0])
                for n in ("dq", "dk", "dv"):
                    errs[f"{name}.{n}"] = rel_err(sl(got[n])[0], ref[n][0])
                if ref["dbias"] is not None:
                    gb = got["dbias"][0][:, a:e, a:e] if name == "packed" else got["dbias"][0]
                    errs[f"{name}.dbias"] = rel_err(gb, ref["dbias"][0])
                errs[f"{name}.out_edges"] = rel_err(sl(got["out"])[0][edge], ref["out"][0][edge])
                errs[f"{name}.dq_edges"] = rel_err(sl(got["dq"])[0][edge], ref["dq"][0][edge])
            print(f"batch row {b} segment [{a}, {e}): " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()),
                  flush=True)
            bad = {k: v for k, v in errs.items() if not v <= tol}
            assert not bad, f"segment [{a}, {e}) of batch row {b}: {bad}"
