"""Full-size checks of the widened forms, in the launch configuration bench.py times.

* packed_varlen with its packing given as k_start and as a dense mask: every output
  bitwise equal to the segment-id run (which test_gpu_workloads.py compares with the
  oracle at full size).
* causal_gqa in the SBHD layout: every output bitwise equal to the BSHD run.
* packed_varlen with a bias broadcast over heads: dbias equals the per-head dbias of the
  same bias expanded over heads, summed over heads in fp32, to the bf16 bar; every other
  output bitwise equal to that run.
* causal_gqa with dropout 0.1, and causal_gqa in fp16: the oracle on sampled (batch row,
  KV head) groups (the last one, with the longest causal rows, and the first).
"""
import numpy as np
import pytest
import torch

import bench
import workloads as W
from harness import TOL, rel_err
from oracle import attention_backward, attention_forward

pytestmark = pytest.mark.gpu


def _run(g, kw):
    import attention_tanh_logit_amd as A
    out, lse, lo = A.attn_fwd(g["q"], g["k"], g["v"], **{k: v for k, v in kw.items() if k != "dq_mode"})
    dq, dk, dv, dbias, dsink = A.attn_bwd(g["q"], g["k"], g["v"], out, lse, g["dout"], out_lo=lo, **kw)
    torch.cuda.synchronize()
    return {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dbias": dbias, "dsink": dsink}


def _same_bits(a, b, names, label):
    for n in names:
        x, y = a[n], b[n]
        if x is None:
            assert y is None, f"{label}: {n} missing on one side"
            continue
        assert torch.equal(x.contiguous().view(torch.int8), y.contiguous().view(torch.int8)), \
            f"{label}: {n} differs bitwise"


@pytest.mark.parametrize("form", ["k_start", "dense_mask"])
def test_packed_forms_bitwise_at_full_size(form):
    w = W.packed_varlen()
    print(f"packed_varlen full size, packing as {form}", flush=True)
    d = W.draw(w)
    g, kw = bench.to_gpu(w, d)
    ref = _run(g, kw)
    g2, kw2 = bench.to_gpu(w, d, form)
    got = _run(g2, kw2)
    _same_bits(ref, got, ["out", "lse", "dq", "dk", "dv", "dbias"], f"packed_varlen as {form}")


def test_sbhd_bitwise_at_full_size():
    w = W.causal_gqa(30.0)
    print("causal_gqa full size, BSHD against SBHD", flush=True)
    d = W.draw(w)
    g, kw = bench.to_gpu(w, d)
    ref = _run(g, kw)
    ws = w.with_(layout="sbhd")
    g2, kw2 = bench.to_gpu(ws, d)
    got = _run(g2, kw2)
    for n in ("out", "dq", "dk", "dv"):
        got[n] = got[n].transpose(0, 1)      # [S, B, H, D] -> [B, S, H, D]
    _same_bits(ref, got, ["out", "lse", "dq", "dk", "dv"], "causal_gqa SBHD")


def test_head_broadcast_dbias_at_full_size():
    w = W.packed_varlen().with_(name="packed_varlen_bias_heads_bf16_cap50", bias_heads=1)
    print("packed_varlen full size, bias broadcast over heads", flush=True)
    d = W.draw(w)
    g, kw = bench.to_gpu(w, d)
    got = _run(g, kw)
    assert got["dbias"].shape == (w.B, 1, w.S, w.S)
    kw_full = dict(kw, bias=kw["bias"].expand(w.B, w.Hq, w.S, w.S).contiguous())
    ref = _run(g, kw_full)
    _same_bits(ref, got, ["out", "lse", "dq", "dk", "dv"], "head-broadcast bias")
    for b in range(w.B):
        acc = torch.zeros((w.S, w.S), dtype=torch.float32, device="cuda")
        for h in range(w.Hq):
            acc += ref["dbias"][b, h].float()
        x = got["dbias"][b, 0].float()
        err = ((x - acc).abs().max() / acc.abs().max()).item()
        print(f"batch row {b}: dbias summed over heads, error {err:.2e}", flush=True)
        assert err <= TOL["bf16"], f"dbias of batch row {b}: {err:.2e}"


@pytest.mark.parametrize("variant", ["dropout", "fp16"])
def test_causal_gqa_variants_match_oracle_on_sampled_groups(variant):
    w = W.causal_gqa(30.0)
    w = w.with_(name="causal_gqa_dropout0.1", dropout_p=0.1) if variant == "dropout" else \
        w.with_(name="causal_gqa_fp16", dtype="fp16")
    print(f"{w.name}: GPU forward + backward", flush=True)
    d = W.draw(w)
    g, kw = bench.to_gpu(w, d)
    got = _run(g, kw)
    G = w.G
    f = lambda x: x.float().cpu().numpy()  # noqa: E731
    okw = dict(softcap=w.softcap, causal=w.causal, window=w.window)
    if w.dropout_p > 0:
        okw.update(dropout_p=w.dropout_p, dropout_seed=w.seed, dropout_offset=0)
    tol = TOL[w.dtype]
    for (b, hk) in [(w.B - 1, w.Hkv - 1), (0, 0)]:
        print(f"{w.name}: oracle on group b={b} kv_head={hk}", flush=True)
        ro, rl = attention_forward(d["q"], d["k"], d["v"], groups=[(b, hk)], **okw)
        rq, rk, rv, _, _ = attention_backward(d["q"], d["k"], d["v"], d["dout"], groups=[(b, hk)], **okw)
        hs = slice(hk * G, (hk + 1) * G)
        errs = {
            "out": rel_err(f(got["out"][b, :, hs]), ro[b, :, hs]),
            "lse": rel_err(f(got["lse"][b, hs]), rl[b, hs]),
            "dq": rel_err(f(got["dq"][b, :, hs]), rq[b, :, hs]),
            "dk": rel_err(f(got["dk"][b, :, hk]), rk[b, :, hk]),
            "dv": rel_err(f(got["dv"][b, :, hk]), rv[b, :, hk]),
        }
        print(f"{w.name} group ({b},{hk}) errors: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
        bad = {k: v for k, v in errs.items() if not v <= tol}
        assert not bad, f"{w.name}: over tolerance {tol}: {bad}"
