"""attn_bwd_noalloc: the backward with the library's static scratch instead of
a caller workspace, checked against attn_bwd on the same inputs.

Both entry points run the same kernels, so with the same dq_mode the results
must agree bit for bit; where "auto" resolves differently (the dU blocks do
not fit the 128 MiB scratch) they must agree to the dtype's bar.  Each test
makes two calls in a row, the second with a smaller problem, so that the
second call runs on scratch the first one left behind.
"""
import numpy as np
import pytest
import torch

import attention_tanh_logit_amd as A
from harness import TOL, as_dense_mask, as_k_start, case, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _inputs(c):
    dt = c["dtype"]
    q, k, v, do = (to_dev(c[n], dt) for n in ("q", "k", "v", "dout"))
    kw = dict(causal=c["causal"], window=c["window"], softcap=c["softcap"], sink_mode=c["sink_mode"])
    if c["sink"] is not None:
        kw["sink"] = torch.from_numpy(c["sink"]).cuda()
    if c["bias"] is not None:
        kw["bias"] = to_dev(c["bias"], dt)
    if c["segment_ids"] is not None:
        kw["segment_ids"] = torch.from_numpy(c["segment_ids"]).cuda()
    if c.get("k_start") is not None:
        kw["k_start"] = torch.from_numpy(np.ascontiguousarray(c["k_start"], dtype=np.int32)).cuda()
    if c.get("mask") is not None:
        kw["mask"] = torch.from_numpy(np.ascontiguousarray(c["mask"], dtype=bool)).cuda()
    if c.get("dropout"):
        kw.update(dropout_p=c["dropout"][0], dropout_seed=c["dropout"][1], dropout_offset=c["dropout"][2])
    return q, k, v, do, kw


def _both(c, mode_ref, mode_noalloc):
    q, k, v, do, kw = _inputs(c)
    out, lse, lo = A.attn_fwd(q, k, v, **kw)
    ref = A.attn_bwd(q, k, v, out, lse, do, out_lo=lo, dq_mode=mode_ref, **kw)
    nan = float("nan")
    outs = {"dq": torch.full_like(q, nan), "dk": torch.full_like(k, nan), "dv": torch.full_like(v, nan)}
    if "bias" in kw:
        outs["dbias"] = torch.full_like(kw["bias"], nan)
    if c["sink_mode"] == "learnable":
        outs["dsink"] = torch.full((q.shape[2],), nan, dtype=torch.float32, device=q.device)
    got = A.ops.attn_bwd_noalloc(q, k, v, out, lse, do, out_lo=lo, dq_mode=mode_noalloc, outputs=outs, **kw)
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dbias", "dsink")
    return ({n: None if t is None else t.float().cpu().numpy() for n, t in zip(names, ref)},
            {n: None if t is None else t.float().cpu().numpy() for n, t in zip(names, got)})


SMALL_AFTER = {
    "bf16_d128": (dict(dtype="bf16", D=128, B=2, S=512, Hq=8, Hkv=2, sink_mode="learnable", bias=True,
                       softcap=50.0, segments=[[100, 301], [64]]),
                  dict(dtype="bf16", D=128, B=1, S=203, Hq=4, Hkv=2, sink_mode="learnable", bias=True,
                       segments=[[77]])),
    "bf16_d64": (dict(dtype="bf16", D=64, B=1, S=1024, Hq=16, Hkv=2, sink_mode="learnable", window=300),
                 dict(dtype="bf16", D=64, B=2, S=130, Hq=4, Hkv=4, sink_mode="learnable")),
    "bf16_d512": (dict(dtype="bf16", D=512, B=1, S=400, Hq=4, Hkv=2, bias=True),
                  dict(dtype="bf16", D=512, B=1, S=70, Hq=2, Hkv=1)),
    "fp32_d256": (dict(dtype="fp32", D=256, B=2, S=300, Hq=4, Hkv=2, sink_mode="learnable", window=64),
                  dict(dtype="fp32", D=256, B=1, S=33, Hq=2, Hkv=2, sink_mode="learnable")),
}


# packed forms and dropout: the first call with a dense mask (its prepared ranges in the
# scratch), the second with k_start
FORMS = {"bf16_d128_dropout_packed": ("dense_mask", "k_start")}
SMALL_AFTER["bf16_d128_dropout_packed"] = (
    dict(dtype="bf16", D=128, B=2, S=512, Hq=8, Hkv=2, dropout_p=0.2, sink_mode="learnable",
         segments=[[100, 301], [64]]),
    dict(dtype="bf16", D=128, B=1, S=203, Hq=4, Hkv=2, dropout_p=0.1, segments=[[77]]))


@pytest.mark.parametrize("name", list(SMALL_AFTER))
def test_noalloc_equals_attn_bwd_bitwise_on_two_calls(name):
    for i, kw in enumerate(SMALL_AFTER[name]):
        c = case(**kw)
        if name in FORMS:
            c = as_dense_mask(c) if FORMS[name][i] == "dense_mask" else as_k_start(c)
        print(f"noalloc {name} call {i + 1}: q={c['q'].shape}", flush=True)
        ref, got = _both(c, "auto", "auto")
        for n, r in ref.items():
            if r is None:
                assert got[n] is None, n
                continue
            assert got[n].tobytes() == r.tobytes(), f"{name} call {i + 1}: {n} differs from attn_bwd"


def test_noalloc_recomputes_where_the_du_blocks_do_not_fit():
    """dU blocks of 4 GiB: attn_bwd "auto" hands them over, attn_bwd_noalloc "auto"
    recomputes (bitwise equal to attn_bwd "recompute", within the bar of "auto");
    then a small call on the same scratch."""
    c = case(dtype="bf16", D=128, B=2, S=8192, Hq=16, Hkv=8, sink_mode="learnable", q_scale=4.0)
    print("noalloc large call", flush=True)
    ref_rec, got = _both(c, "recompute", "auto")
    for n, r in ref_rec.items():
        if r is not None:
            assert got[n].tobytes() == r.tobytes(), f"{n} differs from attn_bwd recompute"
    ref_du, _ = _both(c, "auto", "auto")
    for n, r in ref_du.items():
        if r is not None:
            assert rel_err(got[n], r) <= TOL["bf16"], n
    c2 = case(dtype="bf16", D=128, B=1, S=100, Hq=2, Hkv=1, sink_mode="learnable")
    print("noalloc small call after it", flush=True)
    ref, got = _both(c2, "auto", "auto")
    for n, r in ref.items():
        if r is not None:
            assert got[n].tobytes() == r.tobytes(), f"small call: {n} differs"


def test_noalloc_rejects_a_workspace_beyond_its_scratch():
    c = case(dtype="bf16", D=128, B=1, S=8192, Hq=16, Hkv=8)
    q, k, v, do, kw = _inputs(c)
    out, lse, lo = A.attn_fwd(q, k, v, **kw)
    outs = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v)}
    with pytest.raises(A.AttnError, match="scratch"):
        A.ops.attn_bwd_noalloc(q, k, v, out, lse, do, out_lo=lo, dq_mode="du_blocks", outputs=outs, **kw)
    torch.cuda.synchronize()
