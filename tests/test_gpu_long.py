"""A long causal sequence at the edge of the index ranges: S = 65536 (4.3e9 pairs per head,
8 GiB of dU blocks), checked on what the oracle can compute exactly from a slice.

Under a causal mask the last 64 keys are seen only by the last 64 queries, so the oracle
run on those 64 query rows against all keys (the causal mask written as a dense mask for the
slice) gives exactly: their outputs, lse and dq, and the dk and dv of the last 64 keys.
"""
import numpy as np
import pytest
import torch

import workloads as W
from harness import TOL, rel_err
from oracle import group_backward, group_forward

pytestmark = pytest.mark.gpu


def test_long_causal_sequence_tail_matches_oracle():
    import attention_tanh_logit_amd as A
    S, D, R = 65536, 128, 64
    rng = np.random.default_rng(3)
    f = np.float32
    q = W.round_to_bf16(rng.standard_normal((1, S, 1, D), dtype=f) * f(4.0))
    k = W.round_to_bf16(rng.standard_normal((1, S, 1, D), dtype=f))
    v = W.round_to_bf16(rng.standard_normal((1, S, 1, D), dtype=f))
    do = W.round_to_bf16(rng.standard_normal((1, S, 1, D), dtype=f))
    sink = rng.standard_normal(1, dtype=f) * f(5.0)
    t = lambda x: torch.from_numpy(x).to("cuda", torch.bfloat16)  # noqa: E731
    kw = dict(causal=True, softcap=30.0, sink_mode="learnable", sink=torch.from_numpy(sink).cuda())
    print(f"long causal sequence S={S}: GPU forward + backward", flush=True)
    out, lse, lo = A.attn_fwd(t(q), t(k), t(v), **kw)
    dq, dk, dv, _, dsink = A.attn_bwd(t(q), t(k), t(v), out, lse, t(do), out_lo=lo, **kw)
    torch.cuda.synchronize()
    assert A.ops.bwd_workspace_bytes(t(q), t(k), t(v), **kw) >= 8 << 30    # the dU blocks were used
    rows = np.arange(S - R, S)
    dense = np.arange(S)[None, :] <= rows[:, None]
    okw = dict(softcap=30.0, causal=False, dense=dense, sink=sink)
    print(f"oracle on the last {R} query rows", flush=True)
    ro, rl = group_forward(q[0, S - R:], k[0, :, 0], v[0, :, 0], **okw)
    rq, rk, rv, _, _ = group_backward(q[0, S - R:], k[0, :, 0], v[0, :, 0], do[0, S - R:], **okw)
    g = lambda x: x.float().cpu().numpy()  # noqa: E731
    errs = {
        "out": rel_err(g(out[0, S - R:]), ro),
        "lse": rel_err(g(lse[0, :, S - R:]), rl),
        "dq": rel_err(g(dq[0, S - R:]), rq),
        "dk": rel_err(g(dk[0, S - R:, 0]), rk[S - R:]),
        "dv": rel_err(g(dv[0, S - R:, 0]), rv[S - R:]),
    }
    print("errors: " + ", ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    assert np.isfinite(g(dsink)).all()
    bad = {n: e for n, e in errs.items() if not e <= TOL["bf16"]}
    assert not bad, bad
