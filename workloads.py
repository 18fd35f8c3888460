"""Seeded synthetic inputs for the soft-capped attention workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the fp64 oracle and the HIP path can be fed
from it without sharing any of the method.

Draw order for every workload (one ``numpy.random.default_rng(seed)``):
q, k, v, dO, sink, segment cuts.  The dense additive bias of the packed
workload is drawn per (batch row, query head) slab from
``default_rng([seed, 7919, b, h])`` so that a single slab can be rebuilt
without drawing the whole 4.3 GB tensor.

bf16 (fp16) workloads draw in fp32 and round to nearest-even bf16 (fp16); the
arrays returned here already hold the rounded values (as float32), so the
GPU gets exactly those numbers and the oracle gets them widened to fp64.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


def round_to_fp16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest fp16 (ties to even); returns float32."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs stay below 0xFF800000, so adding at most 0x8000 cannot wrap
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(x.shape)


@dataclasses.dataclass
class Workload:
    """One attention problem: shapes, options and (lazily drawn) inputs."""

    name: str
    dtype: str                  # "bf16" or "fp32"
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    causal: bool = True
    window: int = 0             # <= 0: no sliding window
    softcap: float = 0.0        # 0: cap off
    q_scale: float = 1.0
    sink_mode: str = "none"     # "none" | "off_by_one" | "learnable"
    sink_scale: float = 5.0
    bias_std: float = 0.0       # > 0: dense additive bias [B,Hq,S,S]
    n_segments: Optional[tuple] = None  # (min, max) segments per row: packed rows
    seed: int = 0
    layout: str = "bshd"        # "bshd" or "sbhd" memory layout of q/k/v and their gradients
    dropout_p: float = 0.0      # > 0: attention dropout with seed `seed` and offset 0
    bias_heads: int = 0         # 1: the bias is one [S,S] slab per batch row, broadcast over heads

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def draw(w: Workload, need_dout: bool = True) -> dict:
    """Draw q, k, v, dO, sink and segment ids of workload ``w``.

    Returns float32 numpy arrays in BSHD layout (q/out: [B,S,Hq,D],
    k/v: [B,S,Hkv,D]); ``segment_ids`` int32 [B,S] or None; ``sink`` float32
    [Hq] or None.  The bias is not drawn here (see :func:`bias_slab`).
    """
    rng = np.random.default_rng(w.seed)
    f32 = np.float32
    q = rng.standard_normal((w.B, w.S, w.Hq, w.D), dtype=f32) * f32(w.q_scale)
    k = rng.standard_normal((w.B, w.S, w.Hkv, w.D), dtype=f32)
    v = rng.standard_normal((w.B, w.S, w.Hkv, w.D), dtype=f32)
    do = rng.standard_normal((w.B, w.S, w.Hq, w.D), dtype=f32) if need_dout else None
    sink = None
    if w.sink_mode == "learnable":
        sink = rng.standard_normal(w.Hq, dtype=f32) * f32(w.sink_scale)
    elif w.sink_mode == "off_by_one":
        sink = np.zeros(w.Hq, dtype=f32)
    seg = None
    if w.n_segments is not None:
        seg = _draw_segments(rng, w.B, w.S, *w.n_segments)
    if w.dtype in ("bf16", "fp16"):
        rnd = round_to_bf16 if w.dtype == "bf16" else round_to_fp16
        q, k, v = rnd(q), rnd(k), rnd(v)
        if do is not None:
            do = rnd(do)
    return {"q": q, "k": k, "v": v, "dout": do, "sink": sink, "segment_ids": seg}


def _draw_segments(rng, B: int, S: int, lo: int, hi: int, tile: int = 64) -> np.ndarray:
    """Per row: n ~ U{lo..hi} segments cut at n-1 distinct uniform positions.

    Redrawn (deterministically under the seed) until some cut is not a
    multiple of ``tile`` and the batch holds at least 3 segments, so that
    packing and tile-unaligned boundaries are really exercised.
    """
    while True:
        rows = []
        for _ in range(B):
            n = int(rng.integers(lo, hi + 1))
            cuts = np.sort(rng.choice(np.arange(1, S), size=n - 1, replace=False)) if n > 1 else np.zeros(0, int)
            rows.append(cuts)
        allcuts = np.concatenate(rows) if rows else np.zeros(0)
        nseg = sum(len(c) + 1 for c in rows)
        if nseg >= 3 and np.any(allcuts % tile != 0):
            break
    seg = np.zeros((B, S), dtype=np.int32)
    for b, cuts in enumerate(rows):
        for c in cuts:
            seg[b, c:] += 1
    return seg


def bias_slab(w: Workload, b: int, h: int) -> np.ndarray:
    """The [S,S] additive-bias slab of batch row ``b`` and query head ``h``."""
    rng = np.random.default_rng([w.seed, 7919, b, h])
    x = rng.standard_normal((w.S, w.S), dtype=np.float32) * np.float32(w.bias_std)
    return round_to_bf16(x) if w.dtype == "bf16" else (round_to_fp16(x) if w.dtype == "fp16" else x)


def bias_full(w: Workload) -> np.ndarray:
    """The whole [B,Hq,S,S] bias (use only at sizes that fit in host memory)."""
    out = np.empty((w.B, w.Hq, w.S, w.S), dtype=np.float32)
    for b in range(w.B):
        for h in range(w.Hq):
            out[b, h] = bias_slab(w, b, h)
    return out


def cu_seqlens_from_segments(seg: np.ndarray) -> np.ndarray:
    """Segment ids [B,S] -> cumulative lengths over the flattened token axis."""
    B, S = seg.shape
    starts = [0]
    for b in range(B):
        row = seg[b]
        cut = np.nonzero(np.diff(row))[0] + 1
        for c in cut:
            starts.append(b * S + int(c))
        starts.append((b + 1) * S)
    return np.asarray(starts, dtype=np.int32)


# ---- the five workloads (the first is small enough for the oracle in seconds)

def tiny_fp32() -> Workload:
    return Workload("tiny_fp32_causal_cap30", "fp32", B=1, S=128, Hq=2, Hkv=2, D=64,
                    causal=True, softcap=30.0, q_scale=12.0)


def causal_gqa(softcap: float = 30.0) -> Workload:
    return Workload(f"causal_gqa_bf16_cap{softcap:g}", "bf16", B=4, S=4096, Hq=32, Hkv=8, D=128,
                    causal=True, softcap=softcap, q_scale=4.0)


def packed_varlen() -> Workload:
    return Workload("packed_varlen_bias_bf16_cap50", "bf16", B=2, S=8192, Hq=16, Hkv=8, D=128,
                    causal=True, softcap=50.0, bias_std=0.5, n_segments=(1, 8))


def sink_gqa(sink_mode: str = "learnable", softcap: float = 30.0) -> Workload:
    return Workload(f"sink_{sink_mode}_gqa_bf16_cap{softcap:g}", "bf16", B=1, S=4096, Hq=64, Hkv=8, D=64,
                    causal=True, softcap=softcap, sink_mode=sink_mode)


def window_large_d(D: int = 256, dtype: str = "bf16") -> Workload:
    return Workload(f"window1024_d{D}_{dtype}_cap50", dtype, B=1, S=8192, Hq=8, Hkv=8, D=D,
                    causal=True, window=1024, softcap=50.0, q_scale=6.0)


def all_workloads() -> list:
    """Every sub-run of the five workloads, in order."""
    out = [tiny_fp32(), causal_gqa(30.0), causal_gqa(0.0), packed_varlen()]
    for mode in ("learnable", "off_by_one"):
        for cap in (0.0, 30.0):
            out.append(sink_gqa(mode, cap))
    for D in (256, 512):
        for dt in ("bf16", "fp32"):
            out.append(window_large_d(D, dt))
    return out
