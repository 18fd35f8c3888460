#!/usr/bin/env python
"""Benchmark: fused soft-capped attention forward + backward on one MI355X.

One step = the whole hot path on one batch: attn_fwd (forward kernel) then
the backward's three phases (pre-pass, dk/dv kernel, dq kernel), all on the
current stream with inputs already resident in HBM.  Prints ONE JSON line.

Throughput counts algorithmic work only: 4*D flop per visible (query, key)
pair in the forward and 10*D in the backward (14*D per step), summed over
batch rows and query heads; masked pairs, partial-tile waste and any
recomputation earn nothing.

  python bench.py [--steps K] [--warmup W] [--workload causal_gqa] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
CLOCK_PEAK_BF16 = 256 * 4096 * 2.4e9 / 1e12   # 256 CUs x 4096 flop/clk x 2.4 GHz


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    """sha256 over the code of the HIP sources and the C header (what the counters were
    taken on), with comments and whitespace removed so that a documentation change
    does not retire the counters."""
    import hashlib
    import re
    hsh = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_tanh_logit_amd", "csrc")
    files = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))] + [os.path.join(ROOT, "include", "attn_softcap.h")]
    for f in files:
        with open(f, encoding="utf-8") as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        code = " ".join(code.split())
        hsh.update(os.path.basename(f).encode() + b"\0" + code.encode())
    return hsh.hexdigest()


def measured_traffic(workload_name: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary.

    The summary (profiles/hbm_traffic_<workload>.md) carries one line
    ``bench-traffic: {json}`` with the calibrated FETCH_SIZE + WRITE_SIZE bytes
    per launch and the source digest the counters were taken on; a different
    digest means the kernels changed since, and the traffic is reported as None.
    """
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload_name}.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as fh:
        for line in fh:
            if line.startswith("bench-traffic:"):
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("source_sha256") != kernel_source_digest():
                    return None, "kernels changed since the counters were taken"
                k = rec.get("kernels", {}).get(kernel)
                if k is None:
                    return None, f"no counters for {kernel}"
                return k["fetch_bytes"] + k["write_bytes"], "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"
    return None, "summary has no bench-traffic line"


def calibration_copy(mib: int) -> None:
    """A plain elementwise kernel that reads and writes `mib` MiB each (counter calibration)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def visible_pairs(w, seg=None) -> int:
    """Visible (query, key) pairs per (batch row, query head), summed over batch rows."""
    S, W = w.S, w.window
    if seg is not None:
        total = 0
        for b in range(seg.shape[0]):
            _, counts = __import__("numpy").unique(seg[b], return_counts=True)
            for L in counts:
                L = int(L)
                total += sum(min(i + 1, W) for i in range(L)) if W > 0 else L * (L + 1) // 2
        return total
    per_row = sum(min(i + 1, W) for i in range(S)) if (w.causal and W > 0) else (
        S * (S + 1) // 2 if w.causal else S * S)
    return per_row * w.B


def workload(name):
    import workloads as W
    table = {
        "causal_gqa": W.causal_gqa(30.0),
        "sink_gqa": W.sink_gqa("learnable", 30.0),
        "window_d256": W.window_large_d(256, "bf16"),
        "window_d512": W.window_large_d(512, "bf16"),
        "window_d256_fp32": W.window_large_d(256, "fp32"),
        "window_d512_fp32": W.window_large_d(512, "fp32"),
        "packed_varlen": W.packed_varlen(),
        "packed_varlen_k_start": W.packed_varlen(),
        "packed_varlen_dense_mask": W.packed_varlen(),
        "packed_varlen_bias_heads": W.packed_varlen().with_(name="packed_varlen_bias_heads_bf16_cap50", bias_heads=1),
        "causal_gqa_fp16": W.causal_gqa(30.0).with_(name="causal_gqa_fp16_cap30", dtype="fp16"),
        "causal_gqa_sbhd": W.causal_gqa(30.0).with_(name="causal_gqa_sbhd_bf16_cap30", layout="sbhd"),
        "causal_gqa_dropout": W.causal_gqa(30.0).with_(name="causal_gqa_dropout0.1_bf16_cap30", dropout_p=0.1),
        "sink_gqa_dropout": W.sink_gqa("learnable", 30.0).with_(name="sink_learnable_gqa_dropout0.1_bf16_cap30",
                                                                 dropout_p=0.1),
        "window_d512_dropout": W.window_large_d(512, "bf16").with_(name="window1024_d512_dropout0.1_bf16_cap50",
                                                                    dropout_p=0.1),
        "tiny": W.tiny_fp32(),
    }
    return table[name]


# the packed workload's segments given in the other two packed forms
PACKED_FORMS = {"packed_varlen_k_start": "k_start", "packed_varlen_dense_mask": "dense_mask"}


def to_gpu(w, d, form=None):
    import numpy as np
    import torch
    import workloads as W
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)  # noqa: E731
    lay = (lambda x: x.transpose(0, 1).contiguous()) if w.layout == "sbhd" else (lambda x: x)  # noqa: E731
    g = {"q": lay(t(d["q"])), "k": lay(t(d["k"])), "v": lay(t(d["v"])), "dout": lay(t(d["dout"]))}
    kw = dict(causal=w.causal, window=w.window, softcap=w.softcap, sink_mode=w.sink_mode)
    if w.layout != "bshd":
        kw["layout"] = w.layout
    if w.dropout_p > 0:
        kw.update(dropout_p=w.dropout_p, dropout_seed=w.seed, dropout_offset=0)
    if d["sink"] is not None and w.sink_mode == "learnable":
        kw["sink"] = torch.from_numpy(d["sink"]).cuda()
    seg = d["segment_ids"]
    if seg is not None and form == "k_start":
        # the first token of each token's segment
        ks = np.zeros(seg.shape, dtype=np.int32)
        for b in range(seg.shape[0]):
            starts = np.concatenate([[0], np.nonzero(np.diff(seg[b]))[0] + 1])
            for a, e in zip(starts, list(starts[1:]) + [seg.shape[1]]):
                ks[b, a:e] = a
        kw["k_start"] = torch.from_numpy(ks).cuda()
    elif seg is not None and form == "dense_mask":
        s = torch.from_numpy(seg).cuda()
        kw["mask"] = (s[:, :, None] == s[:, None, :]).contiguous()
    elif seg is not None:
        kw["segment_ids"] = torch.from_numpy(seg).cuda()
    if w.bias_std > 0:
        nh = 1 if w.bias_heads else w.Hq
        bias = torch.empty((w.B, nh, w.S, w.S), dtype=dt, device="cuda")
        for b in range(w.B):
            for h in range(nh):
                bias[b, h] = t(W.bias_slab(w, b, h))
        kw["bias"] = bias
    return g, kw


def run_steps(g, kw, steps, warmup):
    """Warm up, then time exactly `steps` steps; returns (ms_per_step, per-phase ms)."""
    import torch
    import attention_tanh_logit_amd as A
    for _ in range(warmup):
        out, lse, lo = A.attn_fwd(g["q"], g["k"], g["v"], **_fwd_kw(kw))
        A.attn_bwd(g["q"], g["k"], g["v"], out, lse, g["dout"], out_lo=lo, **kw)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        e = ev[s]
        e[0].record()
        out, lse, lo = A.attn_fwd(g["q"], g["k"], g["v"], **_fwd_kw(kw))
        e[1].record()
        A.attn_bwd(g["q"], g["k"], g["v"], out, lse, g["dout"], out_lo=lo, events=e[2:6], **kw)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ph = {"fwd": 0.0, "bwd_pre": 0.0, "dq": 0.0, "dkdv": 0.0}
    for e in ev:
        ph["fwd"] += e[0].elapsed_time(e[1])
        ph["bwd_pre"] += e[2].elapsed_time(e[3])
        ph["dkdv"] += e[3].elapsed_time(e[4])
        ph["dq"] += e[4].elapsed_time(e[5])
    return wall * 1e3 / steps, {k: v / steps for k, v in ph.items()}


def _fwd_kw(kw):
    return {k: v for k, v in kw.items() if k != "dq_mode"}


def dkdv_algorithmic_bytes(w, pairs) -> float:
    """HBM bytes the dk/dv kernel must move at least: Q, dO, K, V read once, dK, dV
    written once, lse and delta read once; with a bias its visible entries read once
    and the dense dbias written once (the workspace hand-off to dq is not counted)."""
    e = 4 if w.dtype == "fp32" else 2
    tok = w.B * w.S
    b = e * tok * w.D * (2 * w.Hq + 4 * w.Hkv) + 8 * tok * w.Hq
    if w.bias_std > 0:
        nh = 1 if w.bias_heads else w.Hq    # a head-broadcast bias (and its dbias) is one slab per batch row
        b += e * pairs * nh // w.Hq + e * w.B * nh * w.S * w.S
    return float(b)


def cpu_baseline(w, d, budget_s=30.0):
    """Time the fp64 oracle (as it stands) on a bounded sample: whole (b, kv-head) groups."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import group_backward, group_forward
    G = w.G
    sink = d["sink"]
    seg = d["segment_ids"]
    done = 0
    flops = 0.0
    t0 = time.perf_counter()
    groups = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    for b, h in groups:
        hs = slice(h * G, (h + 1) * G)
        kw = dict(softcap=w.softcap, causal=w.causal, window=w.window,
                  seg=None if seg is None else seg[b],
                  sink=None if w.sink_mode == "none" else (sink[hs] if sink is not None else np.zeros(G)))
        q, k, v, do = d["q"][b, :, hs], d["k"][b, :, h], d["v"][b, :, h], d["dout"][b, :, hs]
        group_forward(q, k, v, **kw)
        group_backward(q, k, v, do, **kw)
        done += 1
        one = w.with_(B=1)
        flops += 14.0 * w.D * visible_pairs(one, None if seg is None else seg[b:b + 1]) * G
        if time.perf_counter() - t0 > budget_s / 2:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {len(groups)} (batch row, KV head) groups ({done * G} query heads x {w.S} rows), "
                      f"fp64 NumPy forward+backward, {dt:.1f} s; host has {os.cpu_count()} logical CPUs"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="causal_gqa")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cap-ratio", action="store_true")
    ap.add_argument("--no-dq-modes", action="store_true", help="skip the dq_mode=recompute timing")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain copy of this many MiB first (to scale HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the attention path here has no "
              f"multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import attention_tanh_logit_amd as A
    A.lib()
    w = workload(args.workload)
    if args.calib_copy_mib > 0:
        log(f"[bench] calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written")
        calibration_copy(args.calib_copy_mib)
    log(f"[bench] workload {w.name}: drawing inputs")
    d = W.draw(w)
    g, kw = to_gpu(w, d, PACKED_FORMS.get(args.workload))
    pairs = visible_pairs(w, d["segment_ids"]) * w.Hq
    flop_fwd = 4.0 * w.D * pairs
    flop_bwd = 10.0 * w.D * pairs
    flop_step = flop_fwd + flop_bwd
    # dq_mode "auto" takes the dU hand-off (bf16, D = 64/128/256, blocks within 16 GiB):
    # the dq kernel then does only dQ = dU K (2*D per pair); "recompute" redoes S and
    # dP there (6*D per pair; the extra 4*D earn nothing in the step figure)
    ws_auto = A.ops.bwd_workspace_bytes(g["q"], g["k"], g["v"], **kw)
    ws_rec = A.ops.bwd_workspace_bytes(g["q"], g["k"], g["v"], **dict(kw, dq_mode="recompute"))
    du_path = ws_auto != ws_rec
    per_kernel_flop = {"fwd": 4.0 * w.D * pairs, "dq": (2.0 if du_path else 6.0) * w.D * pairs,
                       "dkdv": 8.0 * w.D * pairs}

    log(f"[bench] timing {args.steps} steps after {args.warmup} warmup (dq_mode auto, "
        f"{'dU hand-off' if du_path else 'recompute'}, workspace {ws_auto / 2**30:.2f} GiB)")
    ms, ph = run_steps(g, kw, args.steps, args.warmup)
    log(f"[bench] {ms:.3f} ms/step  phases {ph}")
    peak = PEAK_FP32_TFLOPS if w.dtype == "fp32" else PEAK_BF16_TFLOPS   # fp16 dense MFMA peak = bf16
    value = flop_step / (ms * 1e-3) / 1e12
    fwd_tflops = flop_fwd / (ph["fwd"] * 1e-3) / 1e12
    bwd_ms = ph["bwd_pre"] + ph["dq"] + ph["dkdv"]

    dq_modes = {"auto": {"path": "du_blocks" if du_path else "recompute", "ms_per_step": ms,
                         "kernel_ms": ph, "bwd_workspace_bytes": ws_auto}}
    if du_path and not args.no_dq_modes:
        ms_r, ph_r = run_steps(g, dict(kw, dq_mode="recompute"), args.steps, 1)
        dq_modes["recompute"] = {"path": "recompute", "ms_per_step": ms_r, "kernel_ms": ph_r,
                                 "bwd_workspace_bytes": ws_rec, "tflops": flop_step / (ms_r * 1e-3) / 1e12}
        log(f"[bench] dq_mode recompute: {ms_r:.3f} ms/step, workspace {ws_rec / 2**30:.3f} GiB, phases {ph_r}")

    cap_ratio = None
    if not args.no_cap_ratio and w.softcap > 0:
        kw0 = dict(kw, softcap=0.0)
        ms0, ph0 = run_steps(g, kw0, args.steps, 1)
        bwd0 = ph0["bwd_pre"] + ph0["dq"] + ph0["dkdv"]
        cap_ratio = {"fwd": ph["fwd"] / ph0["fwd"], "bwd": bwd_ms / bwd0,
                     "fwd_bwd": (ph["fwd"] + bwd_ms) / (ph0["fwd"] + bwd0),
                     "uncapped_ms_per_step": ms0}
        log(f"[bench] uncapped {ms0:.3f} ms/step; cap ratio {cap_ratio}")

    dom = max(("fwd", "dq", "dkdv"), key=lambda k: ph[k])
    achieved = per_kernel_flop[dom] / (ph[dom] * 1e-3) / 1e12
    traffic, traffic_src = measured_traffic(args.workload, dom)
    mfma = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "flop_per_launch": per_kernel_flop[dom]}
    if w.bias_std > 0 and dom == "dkdv":
        # the dense dbias write makes the dk/dv kernel HBM-bound on the packed workload
        nbytes = dkdv_algorithmic_bytes(w, pairs)
        gbps = nbytes / (ph[dom] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": gbps / PEAK_HBM_GBPS, "bytes_per_launch": nbytes, "mfma": mfma}
    else:
        roofline = dict(mfma)
    roofline.update({"traffic": traffic, "traffic_source": traffic_src,
                     "traffic_gbps": None if traffic is None else traffic / (ph[dom] * 1e-3) / 1e9,
                     "avg_launch_ms": ph[dom]})

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 CPU oracle on a bounded sample")
        cpu = cpu_baseline(w, d)
        log(f"[bench] cpu baseline {cpu}")

    line = {
        "metric": "attention fwd+bwd TFLOP/s and % of bf16 MFMA peak; capped/uncapped time ratio",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded, workloads.py)",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "causal": w.causal, "window": w.window, "softcap": w.softcap, "sink": w.sink_mode,
                   "bias": w.bias_std > 0, "packed": w.n_segments is not None,
                   "packed_form": PACKED_FORMS.get(args.workload, "segment_ids") if w.n_segments else None,
                   "layout": w.layout, "dropout_p": w.dropout_p, "bias_broadcast_heads": bool(w.bias_heads)},
        "frac_of_peak": value / peak,
        "fwd_tflops": fwd_tflops, "fwd_frac_of_peak": fwd_tflops / peak,
        "bwd_tflops": flop_bwd / (bwd_ms * 1e-3) / 1e12,
        "kernel_ms": ph, "cap_ratio": cap_ratio, "dq_modes": dq_modes,
        "peak_tflops": peak, "peak_tflops_from_clock": CLOCK_PEAK_BF16 if w.dtype != "fp32" else None,
        "algorithmic_flop_per_step": flop_step, "visible_pairs": pairs,
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
