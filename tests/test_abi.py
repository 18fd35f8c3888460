"""The C ABI without a GPU: the library loads, exports every declared symbol, and
fails closed on bad arguments (status code and message, nothing launched).

``attn_validate`` touches no device memory, so these run on the CPU.
"""
import ctypes
import os
import re

import pytest

import attention_tanh_logit_amd as A
from attention_tanh_logit_amd.ops import AttnArgs

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "attn_softcap.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:attn_status|size_t|const char\*)\s+(attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(A.ops.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = A.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def _args(**kw):
    a = AttnArgs()
    a.dtype, a.B, a.Sq, a.Sk, a.Hq, a.Hkv, a.D = 0, 2, 256, 256, 8, 2, 128
    a.q = a.k = a.v = 0x1000
    a.causal, a.window, a.softcap, a.scale, a.sink_mode = 1, 0, 30.0, 0.0, 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _status(a):
    L = A.lib()
    s = L.attn_validate(ctypes.byref(a))
    return s, L.attn_last_error().decode()


def test_valid_arguments_pass():
    assert _status(_args()) == (0, "")
    assert _status(_args(sink_mode=1)) == (0, "")
    assert _status(_args(sink_mode=2, sink=0x2000))[0] == 0
    assert _status(_args(causal=0, Sk=300))[0] == 0
    assert _status(_args(dq_mode=1))[0] == 0
    assert _status(_args(dq_mode=2, dtype=1))[0] == 0
    assert _status(_args(Sq=0, Sk=0))[0] == 0
    assert _status(_args(dtype=2))[0] == 0
    assert _status(_args(dropout_p=0.1, dq_mode=1))[0] == 0          # dropout on the fast dk/dv kernel, D = 128
    assert _status(_args(dropout_p=0.1, dq_mode=1, D=256))[0] == 0
    assert _status(_args(dropout_p=0.1, dq_mode=1, D=64))[0] == 0
    assert _status(_args(dropout_p=0.1, dq_mode=1, D=512))[0] == 0


BAD = {
    "negative_softcap": (dict(softcap=-1.0), 1, "softcap"),
    "nan_softcap": (dict(softcap=float("nan")), 1, "softcap"),
    "inf_softcap": (dict(softcap=float("inf")), 1, "softcap"),
    "gqa_not_divisible": (dict(Hq=6, Hkv=4), 1, "multiple"),
    "head_dim_unsupported": (dict(D=96), 2, "head dim"),
    "learnable_without_sink": (dict(sink_mode=2), 1, "sink"),
    "sink_without_mode": (dict(sink=0x2000), 1, "sink"),
    "off_by_one_with_logits": (dict(sink_mode=1, sink=0x2000), 1, "sink"),
    "bad_sink_mode": (dict(sink_mode=7), 1, "sink_mode"),
    "causal_lengths_differ": (dict(Sk=300), 2, "causal"),
    "segments_and_cu_seqlens": (dict(segment_ids=0x3000, cu_seqlens=0x4000, nseq=2), 1, "not both"),
    "cu_seqlens_batch": (dict(cu_seqlens=0x4000, nseq=2), 1, "B == 1"),
    "cu_seqlens_empty": (dict(B=1, cu_seqlens=0x4000, nseq=0), 1, "nseq"),
    "segments_lengths_differ": (dict(causal=0, Sk=300, segment_ids=0x3000), 1, "Sq == Sk"),
    "bad_dtype": (dict(dtype=5), 1, "dtype"),
    "null_q": (dict(q=None), 1, "NULL"),
    "negative_scale": (dict(scale=-0.1), 1, "scale"),
    "zero_heads": (dict(Hkv=0), 1, "Hkv"),
    "misaligned_q": (dict(q=0x1002), 1, "aligned"),
    "misaligned_bias": (dict(bias=0x2008), 1, "aligned"),
    "bad_dq_mode": (dict(dq_mode=3), 1, "dq_mode"),
    "du_blocks_d512_ragged_bias": (dict(D=512, Sq=250, Sk=250, dq_mode=1, bias=0x2000), 2, "DU_BLOCKS"),
    "du_blocks_ragged_bias": (dict(Sq=250, Sk=250, bias=0x2000, dq_mode=1), 2, "DU_BLOCKS"),
    "keys_empty": (dict(Sk=0, causal=0), 2, "Sk == 0"),
    "bias_bcast_without_bias": (dict(bias_bcast=1), 1, "bias_bcast"),
    "bias_bcast_bad": (dict(bias=0x2000, bias_bcast=4), 1, "bias_bcast"),
    "mask_misaligned": (dict(mask=0x3001), 1, "mask"),
    "dropout_one": (dict(dropout_p=1.0), 1, "dropout_p"),
    "dropout_negative": (dict(dropout_p=-0.1), 1, "dropout_p"),
    "bad_layout": (dict(layout=2), 1, "layout"),
}


@pytest.mark.parametrize("name", list(BAD))
def test_bad_arguments_fail_closed(name):
    kw, code, word = BAD[name]
    s, msg = _status(_args(**kw))
    assert s == code, (s, msg)
    assert word.lower() in msg.lower(), msg


def test_workspace_sizes():
    L = A.lib()
    a = _args()
    assert L.attn_fwd_workspace_size(ctypes.byref(a)) == 0
    assert L.attn_bwd_workspace_size(ctypes.byref(a)) >= 2 * 8 * 256 * 4
    a = _args(segment_ids=0x3000)
    assert L.attn_fwd_workspace_size(ctypes.byref(a)) >= 2 * 2 * 256 * 4
    a = _args(D=96)
    assert L.attn_fwd_workspace_size(ctypes.byref(a)) == ctypes.c_size_t(-1).value


def test_fwd_rejects_before_any_launch():
    """A failing call returns its status without touching the (bogus) pointers."""
    L = A.lib()
    a = _args(softcap=-3.0)
    s = L.attn_fwd(ctypes.byref(a), 0x10, 0x20, None, None, 0, None)
    assert s == 1
    a = _args(sink_mode=2, sink=0x2000)
    s = L.attn_bwd(ctypes.byref(a), 0x10, None, 0x20, 0x30, 0x40, 0x50, 0x60, None, None, None, 1 << 30, None)
    assert s == 1 and "dsink" in L.attn_last_error().decode()


def test_out_lo_is_bf16_only():
    L = A.lib()
    a = _args(dtype=1)
    assert L.attn_fwd(ctypes.byref(a), 0x1000, 0x2000, 0x3000, None, 0, None) == 1
    assert "fp16" in L.attn_last_error().decode()
    s = L.attn_bwd(ctypes.byref(a), 0x1000, 0x3000, 0x2000, 0x4000, 0x5000, 0x6000, 0x7000, None, None, 0x8000,
                   1 << 30, None)
    assert s == 1 and "fp16" in L.attn_last_error().decode()
    a = _args()
    assert L.attn_fwd(ctypes.byref(a), 0x1000, 0x2000, 0x3008, None, 0, None) == 1
    assert "aligned" in L.attn_last_error().decode()


def test_misaligned_outputs_rejected_before_any_launch():
    L = A.lib()
    a = _args()
    assert L.attn_fwd(ctypes.byref(a), 0x1004, 0x2000, None, None, 0, None) == 1
    assert "aligned" in L.attn_last_error().decode()
    s = L.attn_bwd(ctypes.byref(a), 0x1000, None, 0x2000, 0x3000, 0x4002, 0x5000, 0x6000, None, None, 0x7000,
                   1 << 30, None)
    assert s == 1 and "aligned" in L.attn_last_error().decode()


def test_misaligned_workspace_rejected_before_any_launch():
    """The header asks for a 256-byte aligned workspace (its parts are laid out at 256-byte
    offsets from it); a misaligned one is refused with nothing enqueued."""
    L = A.lib()
    a = _args(segment_ids=0x9000)                      # a forward that needs a workspace
    need = L.attn_fwd_workspace_size(ctypes.byref(a))
    assert need > 0
    assert L.attn_fwd(ctypes.byref(a), 0x1000, 0x2000, None, 0x10010, need, None) == 1
    assert "256-byte" in L.attn_last_error().decode()
    need = L.attn_bwd_workspace_size(ctypes.byref(a))
    s = L.attn_bwd(ctypes.byref(a), 0x1000, None, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None, None, 0x10040,
                   need, None)
    assert s == 1 and "256-byte" in L.attn_last_error().decode()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import attention_tanh_logit_amd.ops as ops
    monkeypatch.setattr(ops, "_lib", None)
    monkeypatch.setattr(ops, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        ops.lib()


def test_bwd_workspace_carries_du_blocks_by_dq_mode():
    """bf16: B*Hq*ceil(Sk/32)*ceil(Sq/32) blocks of 2 KiB for dU with dq_mode du_blocks, and
    with auto at D >= 128 while that stays within 16 GiB; none with recompute."""
    L = A.lib()
    a = _args()                       # bf16, B=2, Hq=8, S=256, D=128, dq_mode auto
    with_du = L.attn_bwd_workspace_size(ctypes.byref(a))
    without = L.attn_bwd_workspace_size(ctypes.byref(_args(dq_mode=2)))
    assert with_du - without == 2 * 8 * 8 * 8 * 2048
    assert L.attn_bwd_workspace_size(ctypes.byref(_args(dq_mode=1))) == with_du
    a = _args(Sq=250, Sk=250)         # ragged: still 8 blocks per side
    assert L.attn_bwd_workspace_size(ctypes.byref(a)) - without <= 2 * 8 * 8 * 8 * 2048 + 256
    # auto leaves the hand-off once the blocks pass 16 GiB: B=8, Hq=64, S=16384 needs 32 GiB
    big = dict(B=8, Hq=64, Hkv=8, Sq=16384, Sk=16384)
    auto = L.attn_bwd_workspace_size(ctypes.byref(_args(**big)))
    rec = L.attn_bwd_workspace_size(ctypes.byref(_args(dq_mode=2, **big)))
    forced = L.attn_bwd_workspace_size(ctypes.byref(_args(dq_mode=1, **big)))
    assert auto == rec and forced - rec == 8 * 64 * 512 * 512 * 2048
    d64 = dict(D=64)
    assert L.attn_bwd_workspace_size(ctypes.byref(_args(**d64))) == \
        L.attn_bwd_workspace_size(ctypes.byref(_args(dq_mode=2, **d64)))
    assert L.attn_bwd_workspace_size(ctypes.byref(_args(dq_mode=1, **d64))) - \
        L.attn_bwd_workspace_size(ctypes.byref(_args(dq_mode=2, **d64))) == 2 * 8 * 8 * 8 * 2048
    d512 = dict(D=512)
    assert L.attn_bwd_workspace_size(ctypes.byref(_args(**d512))) - \
        L.attn_bwd_workspace_size(ctypes.byref(_args(dq_mode=2, **d512))) == 2 * 8 * 8 * 8 * 2048
    # fp32: the same blocks in 4-byte elements (4 KiB each), auto from D = 128 on, with a bias or
    # dropout as well (the generic kernels write and read them)
    for extra in ({}, dict(bias=0x2000), dict(dropout_p=0.1), dict(D=512)):
        f32 = dict(dtype=1, **extra)
        assert L.attn_bwd_workspace_size(ctypes.byref(_args(**f32))) - \
            L.attn_bwd_workspace_size(ctypes.byref(_args(dq_mode=2, **f32))) == 2 * 8 * 8 * 8 * 4096, extra
    f64 = dict(dtype=1, D=64)
    assert L.attn_bwd_workspace_size(ctypes.byref(_args(**f64))) == \
        L.attn_bwd_workspace_size(ctypes.byref(_args(dq_mode=2, **f64)))
    assert L.attn_bwd_workspace_size(ctypes.byref(_args(dq_mode=1, **f64))) - \
        L.attn_bwd_workspace_size(ctypes.byref(_args(dq_mode=2, **f64))) == 2 * 8 * 8 * 8 * 4096
    f32 = _args(dtype=1, dq_mode=2)
    g32 = _args(dtype=1, D=256, dq_mode=2)
    # the bf16 run also carries the fp32 dK/dV partials of its head split
    assert L.attn_bwd_workspace_size(ctypes.byref(f32)) == without - _split_partials(_args())
    assert L.attn_bwd_workspace_size(ctypes.byref(g32)) == without - _split_partials(_args())


def _head_split(B, Sk, Hq, Hkv):
    """Smallest divisor s of G = Hq/Hkv with ceil(Sk/128)*Hkv*B*s >= 1024 (else the largest tried)."""
    wgs, G, hs = -(-Sk // 128) * Hkv * B, Hq // Hkv, 1
    for s in range(2, G + 1):
        if wgs * hs >= 1024:
            break
        if G % s == 0:
            hs = s
    return hs


def _split_partials(a):
    hs = _head_split(a.B, a.Sk, a.Hq, a.Hkv)
    n = 2 * hs * a.B * a.Sk * a.Hkv * a.D * 4 if hs > 1 else 0
    return (n + 255) // 256 * 256


def test_bwd_workspace_carries_split_partials_only_for_small_grids():
    """bf16 dk/dv splits a GQA group's query heads over workgroups when the grid is small:
    fp32 partial dK/dV for each split in the workspace; none for a grid of >= 1024 workgroups."""
    L = A.lib()
    for B, S, Hq, Hkv, D, hs in ((2, 256, 8, 2, 128, 4), (1, 4096, 64, 8, 64, 4), (4, 4096, 32, 8, 128, 1),
                                 (1, 4096, 24, 8, 128, 3)):
        assert _head_split(B, S, Hq, Hkv) == hs
        bf = _args(B=B, Sq=S, Sk=S, Hq=Hq, Hkv=Hkv, D=D, dq_mode=2)
        fp = _args(B=B, Sq=S, Sk=S, Hq=Hq, Hkv=Hkv, D=D, dtype=1, dq_mode=2)
        diff = L.attn_bwd_workspace_size(ctypes.byref(bf)) - L.attn_bwd_workspace_size(ctypes.byref(fp))
        assert diff == _split_partials(bf), (B, S, Hq, Hkv, D)


# ---- the binding's own checks: the C ABI sees only pointers, so shapes and devices are checked here

def _t(*shape, dtype=None, device="cpu"):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16, device=device)


MAKE_ARGS_BAD = {
    "k_batch": (lambda: (_t(2, 64, 4, 128), _t(1, 64, 2, 128), _t(1, 64, 2, 128)), {}, "batch"),
    "k_head_dim": (lambda: (_t(2, 64, 4, 128), _t(2, 64, 2, 64), _t(2, 64, 2, 64)), {}, "head dim"),
    "thd_head_dim": (lambda: (_t(64, 4, 128), _t(64, 2, 64), _t(64, 2, 64)),
                     dict(cu_seqlens=_t(3, dtype=__import__("torch").int32)), "head dim"),
    "v_shape": (lambda: (_t(2, 64, 4, 128), _t(2, 64, 2, 128), _t(2, 32, 2, 128)), {}, "same shape"),
    "k_rank": (lambda: (_t(2, 64, 4, 128), _t(64, 2, 128), _t(64, 2, 128)), {}, "BSHD"),
    "sink_on_other_device": (lambda: (_t(2, 64, 4, 128), _t(2, 64, 2, 128), _t(2, 64, 2, 128)),
                             dict(sink_mode="learnable", sink=_t(4, dtype=__import__("torch").float32,
                                                                 device="meta")), "device"),
    "bias_on_other_device": (lambda: (_t(2, 64, 4, 128), _t(2, 64, 2, 128), _t(2, 64, 2, 128)),
                             dict(bias=_t(2, 4, 64, 64, device="meta")), "device"),
    "host_tensors": (lambda: (_t(2, 64, 4, 128), _t(2, 64, 2, 128), _t(2, 64, 2, 128)), {}, "GPU"),
    "bad_dq_mode": (lambda: (_t(2, 64, 4, 128), _t(2, 64, 2, 128), _t(2, 64, 2, 128)),
                    dict(dq_mode="fast"), "dq_mode"),
}


@pytest.mark.parametrize("name", list(MAKE_ARGS_BAD))
def test_make_args_rejects_mismatched_tensors(name):
    mk, kw, word = MAKE_ARGS_BAD[name]
    q, k, v = mk()
    with pytest.raises(ValueError, match=word):
        A.make_args(q, k, v, **kw)


def test_noalloc_rejects_oversize_before_any_launch():
    """attn_bwd_noalloc checks the workspace its problem needs against its 128 MiB
    scratch on the host: explicit dU blocks of 4 GiB are refused with no device call."""
    L = A.lib()
    a = _args(B=4, Sq=4096, Sk=4096, Hq=32, Hkv=8, dq_mode=1)
    s = L.attn_bwd_noalloc(ctypes.byref(a), 0x1000, None, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None, None, None)
    assert s == 2 and "scratch" in L.attn_last_error().decode()
    a = _args(dq_mode=7)
    assert L.attn_bwd_noalloc(ctypes.byref(a), 0x1000, None, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None, None,
                              None) == 1


def test_broadcast_bias_workspace_holds_the_full_gradient():
    L = A.lib()
    full = L.attn_bwd_workspace_size(ctypes.byref(_args(bias=0x2000, dq_mode=2)))
    for f in (1, 2, 3):
        bc = L.attn_bwd_workspace_size(ctypes.byref(_args(bias=0x2000, bias_bcast=f, dq_mode=2)))
        assert bc - full == 2 * 8 * 256 * 256 * 2     # B*Hq*Sq*Sk bf16


def test_make_args_broadcast_bias_flags():
    import torch
    q = _t(2, 64, 4, 128)
    k = _t(2, 64, 2, 128)
    for shape, flags in (((2, 4, 64, 64), 0), ((1, 4, 64, 64), 1), ((2, 1, 64, 64), 2), ((1, 1, 64, 64), 3)):
        with pytest.raises(ValueError, match="GPU"):       # shapes pass; the host tensors are then refused
            A.make_args(q, k, k, bias=_t(*shape))
    with pytest.raises(ValueError, match="bias must be"):
        A.make_args(q, k, k, bias=_t(3, 4, 64, 64))


def test_ctypes_struct_matches_the_c_header(tmp_path):
    """attn_args as the C compiler lays it out (gcc on the header) equals the binding's ctypes struct."""
    import subprocess
    names = [f[0] for f in AttnArgs._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "attn_softcap.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(attn_args));\n' +
                   "".join(f'  printf("%zu\\n", offsetof(attn_args, {n}));\n' for n in names) + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)])
    out = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    assert out[0] == ctypes.sizeof(AttnArgs)
    assert out[1:] == [getattr(AttnArgs, n).offset for n in names]
