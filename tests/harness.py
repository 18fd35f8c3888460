"""Shared test plumbing: seeded inputs, the GPU call, the oracle call, the metric.

The GPU side goes through ``attention_tanh_logit_amd`` (the C ABI); the
reference side through ``oracle`` (fp64 NumPy).  Both get the same seeded
values: bf16 inputs are drawn in fp32, rounded to bf16, and the oracle sees
those rounded values widened to fp64.

Error metric (normwise, per output tensor): max|x - ref| / max|ref|.
Tolerances: fp32 path 1e-5, bf16 path 1e-2, fp16 path 2e-3.  The fp16 bar is
derived from the bf16 one: both paths round the same quantities (inputs,
probabilities and dS before the matrix products, the outputs) to a 16-bit
type, and the bf16 path's worst normwise error is about 1.6 of its unit
roundoff 2^-8; fp16's unit roundoff is 2^-11, so its errors are 8x smaller,
about 8e-4, and the bar keeps a factor 2.5 over that.
"""
from __future__ import annotations

import numpy as np
import torch

import workloads as W
from oracle import attention_backward, attention_forward

TOL = {"fp32": 1e-5, "bf16": 1e-2, "fp16": 2e-3}


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    fin = np.isfinite(ref)
    if not np.array_equal(fin, np.isfinite(x)):
        return float("inf")
    if not np.array_equal(np.where(fin, 0, ref), np.where(fin, 0, x)):   # same infinities
        return float("inf")
    d = np.abs(np.where(fin, x, 0.0) - np.where(fin, ref, 0.0)).max()
    s = np.abs(np.where(fin, ref, 0.0)).max()
    return float(d / s) if s > 0 else float(d)


def tdtype(dtype: str):
    return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]


def round_to_fp16(x):
    """Round float32 values to the nearest fp16 (ties to even); returns float32."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def to_dev(x, dtype: str, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=tdtype(dtype))


def case(dtype="bf16", B=2, S=200, Hq=4, Hkv=2, D=64, causal=True, window=0, softcap=30.0, q_scale=4.0,
         sink_mode="none", bias=False, segments=None, seed=0, Sk=None, bias_bcast="", dropout_p=0.0):
    """Random inputs for one case (numpy fp32 values, bf16-rounded for bf16)."""
    rng = np.random.default_rng(seed)
    Sk = S if Sk is None else Sk
    f = np.float32
    q = rng.standard_normal((B, S, Hq, D), dtype=f) * f(q_scale)
    k = rng.standard_normal((B, Sk, Hkv, D), dtype=f)
    v = rng.standard_normal((B, Sk, Hkv, D), dtype=f)
    do = rng.standard_normal((B, S, Hq, D), dtype=f)
    sink = None
    if sink_mode == "learnable":
        sink = rng.standard_normal(Hq, dtype=f) * f(5.0)
    # bias_bcast: "batch" and/or "heads" give the bias a 1 in that dimension (broadcast)
    bshape = (1 if "batch" in bias_bcast else B, 1 if "heads" in bias_bcast else Hq, S, Sk)
    b = rng.standard_normal(bshape, dtype=f) * f(0.5) if bias else None
    seg = None
    if segments is not None:
        seg = np.zeros((B, S), dtype=np.int32)
        for bb in range(B):
            for c in segments[bb % len(segments)]:
                seg[bb, c:] += 1
    if dtype in ("bf16", "fp16"):
        rnd = W.round_to_bf16 if dtype == "bf16" else round_to_fp16
        q, k, v, do = (rnd(x) for x in (q, k, v, do))
        if b is not None:
            b = rnd(b)
    return dict(dtype=dtype, q=q, k=k, v=v, dout=do, sink=sink, sink_mode=sink_mode, bias=b, segment_ids=seg,
                causal=causal, window=window, softcap=softcap, k_start=None, mask=None,
                dropout=(dropout_p, 0x1234_5678_9ABC_DEF0 + seed, 3 + seed) if dropout_p else None)


def as_k_start(c):
    """The case's packing written as k_start (first key of each token's segment) instead of ids."""
    seg = c["segment_ids"]
    ks = np.zeros(seg.shape, dtype=np.int32)
    for b in range(seg.shape[0]):
        starts = np.concatenate([[0], np.nonzero(np.diff(seg[b]))[0] + 1])
        for a, e in zip(starts, list(starts[1:]) + [seg.shape[1]]):
            ks[b, a:e] = a
    return dict(c, segment_ids=None, k_start=ks)


def as_dense_mask(c):
    """The case's packing written as a dense boolean mask (same segment) instead of ids."""
    seg = c["segment_ids"]
    return dict(c, segment_ids=None, mask=seg[:, :, None] == seg[:, None, :])


def run_gpu(c, backward=True, thd=False, dq_mode="auto", residual=True, layout="bshd", nan_after_bias=False):
    """The case through the C ABI; results as numpy in BSHD order.  layout="sbhd"
    hands the library [S, B, H, D] tensors (and transposes the results back).
    nan_after_bias: the bias sits at the start of a larger buffer whose tail is NaN,
    so that a read past the bias's last element shows."""
    import attention_tanh_logit_amd as A
    dt = c["dtype"]
    sb = layout == "sbhd"
    lay = (lambda x: x.transpose(0, 1).contiguous()) if sb else (lambda x: x)  # noqa: E731
    q, k, v = (lay(to_dev(c[n], dt)) for n in ("q", "k", "v"))
    kw = dict(causal=c["causal"], window=c["window"], softcap=c["softcap"], sink_mode=c["sink_mode"])
    if sb:
        kw["layout"] = "sbhd"
    if c.get("dropout"):
        kw.update(dropout_p=c["dropout"][0], dropout_seed=c["dropout"][1], dropout_offset=c["dropout"][2])
    if c["sink"] is not None:
        kw["sink"] = torch.from_numpy(c["sink"]).cuda()
    if c["bias"] is not None:
        kw["bias"] = to_dev(c["bias"], dt)
        if nan_after_bias:
            n = kw["bias"].numel()
            buf = torch.full((n + 8192,), float("nan"), dtype=kw["bias"].dtype, device=kw["bias"].device)
            buf[:n] = kw["bias"].reshape(-1)
            kw["bias"] = buf[:n].view(kw["bias"].shape)
    if thd:
        assert c["segment_ids"] is not None and c["segment_ids"].shape[0] == 1 or c.get("k_start") is None
        cu = W.cu_seqlens_from_segments(c["segment_ids"])
        kw["cu_seqlens"] = torch.from_numpy(cu).cuda()
        q, k, v = (x.reshape(-1, *x.shape[2:]) for x in (q, k, v))
    elif c["segment_ids"] is not None:
        kw["segment_ids"] = torch.from_numpy(c["segment_ids"]).cuda()
    if c.get("k_start") is not None:
        ks = torch.from_numpy(np.ascontiguousarray(c["k_start"], dtype=np.int32)).cuda()
        kw["k_start"] = ks.reshape(-1) if thd else ks
    if c.get("mask") is not None:
        mk = torch.from_numpy(np.ascontiguousarray(c["mask"], dtype=bool)).cuda()
        kw["mask"] = mk[0] if thd else mk
    # results land in NaN-filled buffers, so an element the kernels leave unwritten shows up
    nan = float("nan")
    B_, S_ = c["q"].shape[:2]
    lse_shape = (q.shape[1], q.shape[0]) if thd else (B_, q.shape[2], S_)
    out, lse, out_lo = A.attn_fwd(q, k, v, out=torch.full_like(q, nan),
                                  lse=torch.full(lse_shape, nan, dtype=torch.float32, device=q.device),
                                  residual=residual, **kw)
    res = {"out": out, "lse": lse}
    if backward:
        do = lay(to_dev(c["dout"], dt))
        if thd:
            do = do.reshape(-1, *do.shape[2:])
        outs = {"dq": torch.full_like(q, nan), "dk": torch.full_like(k, nan), "dv": torch.full_like(v, nan)}
        if "bias" in kw:
            outs["dbias"] = torch.full_like(kw["bias"], nan)
        dq, dk, dv, dbias, dsink = A.attn_bwd(q, k, v, out, lse, do, out_lo=out_lo, outputs=outs, dq_mode=dq_mode,
                                              **kw)
        res.update(dq=dq, dk=dk, dv=dv, dbias=dbias, dsink=dsink)
    torch.cuda.synchronize()
    if sb:
        for n in ("out", "dq", "dk", "dv"):
            if res.get(n) is not None:
                res[n] = res[n].transpose(0, 1)
    res = {n: (None if t is None else t.float().cpu().numpy()) for n, t in res.items()}
    if thd:  # back to the BSHD view of the same rows
        B, S = c["q"].shape[:2]
        for n in ("out", "dq", "dk", "dv"):
            if res.get(n) is not None:
                res[n] = res[n].reshape(B, S, *res[n].shape[1:])
        res["lse"] = res["lse"].reshape(-1, B, S).transpose(1, 0, 2)
    return res


def run_oracle(c, backward=True, groups=None):
    kw = dict(causal=c["causal"], window=c["window"], softcap=c["softcap"], bias=c["bias"],
              segment_ids=c["segment_ids"], sink=c["sink"] if c["sink_mode"] == "learnable"
              else (np.zeros(c["q"].shape[2]) if c["sink_mode"] == "off_by_one" else None), groups=groups,
              k_start=c.get("k_start"), mask=c.get("mask"))
    if c.get("dropout"):
        kw.update(dropout_p=c["dropout"][0], dropout_seed=c["dropout"][1], dropout_offset=c["dropout"][2])
    out, lse = attention_forward(c["q"], c["k"], c["v"], **kw)
    res = {"out": out, "lse": lse}
    if backward:
        dq, dk, dv, dbias, dsink = attention_backward(c["q"], c["k"], c["v"], c["dout"], **kw)
        res.update(dq=dq, dk=dk, dv=dv, dbias=dbias, dsink=dsink if c["sink_mode"] == "learnable" else None)
    return res


# the head axis of each output tensor (query heads, or KV heads for dk/dv)
HEAD_AXIS = {"out": 2, "dq": 2, "dk": 2, "dv": 2, "lse": 1, "dbias": 1}


def per_head_errors(g, r, axis):
    """Normwise error of every (batch row, head) slice: {(b, h): err}."""
    out = {}
    for b in range(r.shape[0]):
        for h in range(r.shape[axis]):
            idx = [b] + [slice(None)] * (r.ndim - 1)
            idx[axis] = h
            out[(b, h)] = rel_err(g[tuple(idx)], r[tuple(idx)])
    return out


def compare(gpu, ref, dtype, names=("out", "lse", "dq", "dk", "dv", "dbias", "dsink"), per_head=False):
    """Normwise errors per tensor; returns {name: err}.

    With per_head, tensors with a head axis also get one error per
    (batch row, head) slice, reported under "name[b,h]" keys, so that a
    single bad head shows up even when the whole tensor's error is small.
    """
    errs = {}
    for n in names:
        if ref.get(n) is None:
            assert gpu.get(n) is None, f"{n}: GPU produced a tensor the oracle did not"
            continue
        g = gpu[n]
        r = ref[n]
        assert g.shape == r.shape, f"{n}: shape {g.shape} vs {r.shape}"
        errs[n] = rel_err(g, r)
        if per_head and n in HEAD_AXIS and r.ndim >= 3:
            for (b, h), e in per_head_errors(g, r, HEAD_AXIS[n]).items():
                errs[f"{n}[{b},{h}]"] = e
    return errs
