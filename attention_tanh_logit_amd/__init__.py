"""MI355X-native fused attention with tanh logit soft-capping and a softmax sink.

The compute path is the gfx950 HIP library ``libattn_softcap.so`` behind the C
ABI in ``include/attn_softcap.h``; this package only marshals arguments.
"""
from .ops import AttnError, attn_bwd, attn_fwd, lib, make_args  # noqa: F401

__all__ = ["attn_fwd", "attn_bwd", "AttnError", "lib", "make_args"]
