"""Thin Python binding over the C ABI in ``include/attn_softcap.h``.

Argument marshalling only: tensors are passed as raw device pointers with the
current HIP stream, every step of the computation runs in the HIP library,
and a missing library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_softcap.so")

ATTN_OK, ATTN_INVALID_ARGUMENT, ATTN_UNSUPPORTED, ATTN_HIP_ERROR = 0, 1, 2, 3
ATTN_BF16, ATTN_FP32, ATTN_FP16 = 0, 1, 2
SINK_MODES = {"none": 0, "off_by_one": 1, "learnable": 2}
DQ_MODES = {"auto": 0, "du_blocks": 1, "recompute": 2}
LAYOUTS = {"bshd": 0, "sbhd": 1}


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("B", ctypes.c_int), ("Sq", ctypes.c_int), ("Sk", ctypes.c_int),
        ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("D", ctypes.c_int),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("segment_ids", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("nseq", ctypes.c_int),
        ("causal", ctypes.c_int),
        ("window", ctypes.c_int),
        ("softcap", ctypes.c_float),
        ("scale", ctypes.c_float),
        ("sink_mode", ctypes.c_int),
        ("sink", ctypes.c_void_p),
        ("dq_mode", ctypes.c_int),
        ("k_start", ctypes.c_void_p),
        ("mask", ctypes.c_void_p),
        ("bias_bcast", ctypes.c_int),
        ("layout", ctypes.c_int),
        ("dropout_p", ctypes.c_float),
        ("dropout_seed", ctypes.c_uint64),
        ("dropout_offset", ctypes.c_uint64),
    ]


EXPORTS = ("attn_validate", "attn_fwd_workspace_size", "attn_bwd_workspace_size",
           "attn_fwd", "attn_bwd", "attn_bwd_pre", "attn_bwd_dq", "attn_bwd_dkdv", "attn_bwd_noalloc",
           "attn_last_error")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"attn status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m attention_tanh_logit_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(AttnArgs)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.attn_validate.argtypes = [P]
    L.attn_validate.restype = ctypes.c_int
    L.attn_fwd_workspace_size.argtypes = [P]
    L.attn_fwd_workspace_size.restype = sz
    L.attn_bwd_workspace_size.argtypes = [P]
    L.attn_bwd_workspace_size.restype = sz
    L.attn_fwd.argtypes = [P, vp, vp, vp, vp, sz, vp]
    L.attn_fwd.restype = ctypes.c_int
    L.attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.attn_bwd.restype = ctypes.c_int
    L.attn_bwd_pre.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.attn_bwd_pre.restype = ctypes.c_int
    L.attn_bwd_dq.argtypes = [P, vp, vp, vp, vp, sz, vp]
    L.attn_bwd_dq.restype = ctypes.c_int
    L.attn_bwd_dkdv.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    L.attn_bwd_dkdv.restype = ctypes.c_int
    L.attn_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.attn_bwd_noalloc.restype = ctypes.c_int
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(status: int) -> None:
    if status != ATTN_OK:
        raise AttnError(status, lib().attn_last_error().decode())


def make_args(q, k, v, *, bias=None, segment_ids=None, cu_seqlens=None, causal=False, window=0,
              softcap=0.0, scale=0.0, sink_mode="none", sink=None, dq_mode="auto", k_start=None,
              mask=None, layout="bshd", dropout_p=0.0, dropout_seed=0, dropout_offset=0) -> AttnArgs:
    """Fill the C argument struct from tensors (BSHD or SBHD, or THD with cu_seqlens).

    The C ABI sees only pointers and sizes, so every shape, dtype and device
    check the kernels rely on happens here: k and v must match q's batch and
    head dim, every tensor must be contiguous and on q's device, and that
    device must be a GPU.  Violations raise ValueError / TypeError before
    anything reaches the library.
    """
    thd = cu_seqlens is not None
    if thd:
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("THD layout: q, k, v must be [T, H, D]")
        B, Sq, Hq, D = 1, q.shape[0], q.shape[1], q.shape[2]
        Sk, Hkv = k.shape[0], k.shape[1]
    elif layout == "sbhd":
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("SBHD layout: q, k, v must be [S, B, H, D]")
        Sq, B, Hq, D = q.shape
        Sk, Hkv = k.shape[0], k.shape[2]
        if k.shape[1] != B:
            raise ValueError(f"k has batch {k.shape[1]}, q has {B}")
    else:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("BSHD layout: q, k, v must be [B, S, H, D]")
        B, Sq, Hq, D = q.shape
        Sk, Hkv = k.shape[1], k.shape[2]
        if k.shape[0] != B:
            raise ValueError(f"k has batch {k.shape[0]}, q has {B}")
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    if k.shape[-1] != D:
        raise ValueError(f"k has head dim {k.shape[-1]}, q has {D}")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if q.dtype == torch.bfloat16:
        dt = ATTN_BF16
    elif q.dtype == torch.float16:
        dt = ATTN_FP16
    elif q.dtype == torch.float32:
        dt = ATTN_FP32
    else:
        raise TypeError("q must be bfloat16, float16 or float32")
    for name, t in (("k", k), ("v", v), ("bias", bias)):
        if t is not None and t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype")
    tensors = (("q", q), ("k", k), ("v", v), ("bias", bias), ("segment_ids", segment_ids),
               ("cu_seqlens", cu_seqlens), ("sink", sink), ("k_start", k_start), ("mask", mask))
    for name, t in tensors:
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    bias_bcast = 0
    if bias is not None:
        if bias.dim() != 4 or tuple(bias.shape[2:]) != (Sq, Sk) or bias.shape[0] not in (1, B) \
                or bias.shape[1] not in (1, Hq):
            raise ValueError(f"bias must be [B or 1, Hq or 1, Sq, Sk] with B, Hq, Sq, Sk = {(B, Hq, Sq, Sk)}")
        bias_bcast = (1 if bias.shape[0] != B else 0) | (2 if bias.shape[1] != Hq else 0)
    if segment_ids is not None and (segment_ids.dtype != torch.int32 or tuple(segment_ids.shape) != (B, Sq)):
        raise ValueError("segment_ids must be int32 [B, Sq]")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1):
        raise ValueError("cu_seqlens must be int32 [nseq + 1]")
    if sink is not None and (sink.dtype != torch.float32 or tuple(sink.shape) != (Hq,)):
        raise ValueError("sink must be float32 [Hq]")
    if k_start is not None and (k_start.dtype != torch.int32 or
                                tuple(k_start.shape) != ((Sq,) if thd else (B, Sq))):
        raise ValueError("k_start must be int32 [B, Sq] ([T] for THD)")
    if mask is not None and (mask.dtype not in (torch.bool, torch.uint8) or
                             tuple(mask.shape) != ((Sq, Sk) if thd else (B, Sq, Sk))):
        raise ValueError("mask must be bool or uint8 [B, Sq, Sk] ([T, T] for THD)")
    for name, t in tensors[1:]:
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}: every tensor must be on q's device")
    if sink_mode not in SINK_MODES:
        raise ValueError(f"sink_mode must be one of {sorted(SINK_MODES)}")
    if dq_mode not in DQ_MODES:
        raise ValueError(f"dq_mode must be one of {sorted(DQ_MODES)}")
    if q.device.type != "cuda":
        raise ValueError(f"q is on {q.device}: the library takes GPU tensors only")
    a = AttnArgs()
    a.dtype = dt
    a.B, a.Sq, a.Sk, a.Hq, a.Hkv, a.D = B, Sq, Sk, Hq, Hkv, D
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.bias = _ptr(bias)
    a.segment_ids = _ptr(segment_ids)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.nseq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    a.causal = int(bool(causal))
    a.window = int(window)
    a.softcap = float(softcap)
    a.scale = float(scale)
    a.sink_mode = SINK_MODES[sink_mode]
    a.sink = _ptr(sink)
    a.dq_mode = DQ_MODES[dq_mode]
    a.k_start = _ptr(k_start)
    a.mask = _ptr(mask)
    a.bias_bcast = bias_bcast
    a.layout = LAYOUTS[layout]
    a.dropout_p = float(dropout_p)
    a.dropout_seed = int(dropout_seed) & 0xFFFFFFFFFFFFFFFF
    a.dropout_offset = int(dropout_offset) & 0xFFFFFFFFFFFFFFFF
    return a


def _like(name, t, like):
    if t.shape != like.shape or t.dtype != like.dtype or t.device != like.device or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous with the shape, dtype and device of {like.shape} {like.dtype}")
    return t


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def attn_fwd(q, k, v, *, bias=None, segment_ids=None, cu_seqlens=None, causal=False, window=0, softcap=0.0,
             scale=0.0, sink_mode="none", sink=None, k_start=None, mask=None, layout="bshd", dropout_p=0.0,
             dropout_seed=0, dropout_offset=0, out=None, lse=None, out_lo=None, residual=True):
    """Forward: returns (out, lse, out_lo); lse is float32 [B, Hq, Sq] ([Hq, T] for THD).

    out_lo (bf16 and fp16; None for fp32 or with ``residual=False``) is the
    part of the fp32 output that ``out`` drops in its rounding; hand it to
    :func:`attn_bwd` so that delta = <dO, O> is taken from the fp32 output.
    """
    L = lib()
    a = make_args(q, k, v, bias=bias, segment_ids=segment_ids, cu_seqlens=cu_seqlens, causal=causal,
                  window=window, softcap=softcap, scale=scale, sink_mode=sink_mode, sink=sink, k_start=k_start,
                  mask=mask, layout=layout,
                  dropout_p=dropout_p, dropout_seed=dropout_seed, dropout_offset=dropout_offset)
    _check(L.attn_validate(ctypes.byref(a)))
    shape = (a.Hq, a.Sq) if cu_seqlens is not None else (a.B, a.Hq, a.Sq)
    out = torch.empty_like(q) if out is None else _like("out", out, q)
    if lse is None:
        lse = torch.empty(shape, dtype=torch.float32, device=q.device)
    elif tuple(lse.shape) != shape or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise ValueError(f"lse must be contiguous float32 {list(shape)}")
    if a.dtype != ATTN_FP32 and (residual or out_lo is not None):
        out_lo = torch.empty_like(q) if out_lo is None else _like("out_lo", out_lo, q)
    elif out_lo is not None:
        raise ValueError("out_lo is for bf16 and fp16 outputs only")
    nws = L.attn_fwd_workspace_size(ctypes.byref(a))
    ws = _workspace(nws, q.device)
    _check(L.attn_fwd(ctypes.byref(a), _ptr(out), _ptr(lse), _ptr(out_lo), _ptr(ws), nws, _stream(q)))
    return out, lse, out_lo


def attn_bwd(q, k, v, out, lse, dout, *, out_lo=None, bias=None, segment_ids=None, cu_seqlens=None, causal=False,
             window=0, softcap=0.0, scale=0.0, sink_mode="none", sink=None, dq_mode="auto", k_start=None, mask=None,
             layout="bshd", dropout_p=0.0, dropout_seed=0, dropout_offset=0, want_dbias=None, events=None,
             outputs=None):
    """Backward: returns (dq, dk, dv, dbias or None, dsink or None).

    ``out_lo`` is what :func:`attn_fwd` returned beside ``out`` (bf16; None
    takes delta from ``out`` alone).  ``dq_mode`` picks how dq is formed:
    "auto", "du_blocks" or "recompute" (see ``attn_dq_mode`` in the header).
    With ``events`` (four torch.cuda.Event) the three phases are launched
    through their own entry points (pre-pass, dk/dv, dq, in that order) with
    an event recorded before the pre-pass and after each phase, on the
    current stream.  ``outputs`` may hold preallocated result tensors under
    "dq", "dk", "dv", "dbias", each contiguous with the shape, dtype and
    device of q, k, v, bias; every element of each is overwritten.
    """
    L = lib()
    a = make_args(q, k, v, bias=bias, segment_ids=segment_ids, cu_seqlens=cu_seqlens, causal=causal,
                  window=window, softcap=softcap, scale=scale, sink_mode=sink_mode, sink=sink, dq_mode=dq_mode,
                  k_start=k_start, mask=mask, layout=layout,
                  dropout_p=dropout_p, dropout_seed=dropout_seed, dropout_offset=dropout_offset)
    _check(L.attn_validate(ctypes.byref(a)))
    _like("out", out, q)
    _like("dout", dout, q)
    if out_lo is not None:
        _like("out_lo", out_lo, q)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != a.B * a.Hq * a.Sq \
            or lse.device != q.device:
        raise ValueError("lse must be contiguous float32 [B, Hq, Sq] on q's device")
    want_dbias = (bias is not None) if want_dbias is None else want_dbias
    given = outputs or {}
    unknown = set(given) - {"dq", "dk", "dv", "dbias"}
    if unknown:
        raise ValueError(f"unknown outputs: {sorted(unknown)}")

    def result(name, like):
        t = given.get(name)
        return torch.empty_like(like) if t is None else _like(f"outputs[{name!r}]", t, like)

    dq = result("dq", q)
    dk = result("dk", k)
    dv = result("dv", v)
    dbias = result("dbias", bias) if (want_dbias and bias is not None) else None
    dsink = torch.empty(a.Hq, dtype=torch.float32, device=q.device) if sink_mode == "learnable" else None
    nws = L.attn_bwd_workspace_size(ctypes.byref(a))
    ws = _workspace(nws, q.device)
    st = _stream(q)
    if events is None:
        _check(L.attn_bwd(ctypes.byref(a), _ptr(out), _ptr(out_lo), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                          _ptr(dv), _ptr(dbias), _ptr(dsink), _ptr(ws), nws, st))
    else:
        events[0].record()
        _check(L.attn_bwd_pre(ctypes.byref(a), _ptr(out), _ptr(out_lo), _ptr(lse), _ptr(dout), _ptr(dbias),
                              _ptr(dsink), _ptr(ws), nws, st))
        events[1].record()
        _check(L.attn_bwd_dkdv(ctypes.byref(a), _ptr(lse), _ptr(dout), _ptr(dk), _ptr(dv), _ptr(dbias),
                               _ptr(ws), nws, st))
        events[2].record()
        _check(L.attn_bwd_dq(ctypes.byref(a), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(ws), nws, st))
        events[3].record()
    return dq, dk, dv, dbias, dsink


def attn_bwd_noalloc(q, k, v, out, lse, dout, *, out_lo=None, bias=None, segment_ids=None, cu_seqlens=None,
                     causal=False, window=0, softcap=0.0, scale=0.0, sink_mode="none", sink=None, dq_mode="auto",
                     k_start=None, mask=None, layout="bshd", dropout_p=0.0, dropout_seed=0, dropout_offset=0,
                     outputs):
    """The backward through ``attn_bwd_noalloc``: no workspace, the library's own
    static scratch instead.  ``outputs`` must hold preallocated "dq", "dk", "dv"
    (and "dbias" with a bias, "dsink" with a learnable sink) tensors, each
    contiguous with the shape, dtype and device of its input; this function
    allocates nothing on the device.  Returns (dq, dk, dv, dbias, dsink)."""
    L = lib()
    a = make_args(q, k, v, bias=bias, segment_ids=segment_ids, cu_seqlens=cu_seqlens, causal=causal,
                  window=window, softcap=softcap, scale=scale, sink_mode=sink_mode, sink=sink, dq_mode=dq_mode,
                  k_start=k_start, mask=mask, layout=layout,
                  dropout_p=dropout_p, dropout_seed=dropout_seed, dropout_offset=dropout_offset)
    _check(L.attn_validate(ctypes.byref(a)))
    _like("out", out, q)
    _like("dout", dout, q)
    if out_lo is not None:
        _like("out_lo", out_lo, q)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != a.B * a.Hq * a.Sq \
            or lse.device != q.device:
        raise ValueError("lse must be contiguous float32 [B, Hq, Sq] on q's device")
    dq = _like("outputs['dq']", outputs["dq"], q)
    dk = _like("outputs['dk']", outputs["dk"], k)
    dv = _like("outputs['dv']", outputs["dv"], v)
    dbias = _like("outputs['dbias']", outputs["dbias"], bias) if outputs.get("dbias") is not None else None
    dsink = None
    if sink_mode == "learnable":
        dsink = outputs["dsink"]
        if tuple(dsink.shape) != (a.Hq,) or dsink.dtype != torch.float32 or dsink.device != q.device \
                or not dsink.is_contiguous():
            raise ValueError("outputs['dsink'] must be contiguous float32 [Hq] on q's device")
    _check(L.attn_bwd_noalloc(ctypes.byref(a), _ptr(out), _ptr(out_lo), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                              _ptr(dv), _ptr(dbias), _ptr(dsink), _stream(q)))
    return dq, dk, dv, dbias, dsink


def bwd_workspace_bytes(q, k, v, **kw) -> int:
    """attn_bwd_workspace_size for these tensors and options (the bench reports it)."""
    a = make_args(q, k, v, **kw)
    _check(lib().attn_validate(ctypes.byref(a)))
    return int(lib().attn_bwd_workspace_size(ctypes.byref(a)))
