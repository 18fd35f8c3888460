"""Plain fp64 CPU oracle for soft-capped attention with a softmax sink.

Test infrastructure only: the tests, the package's smoke check and the
bench's CPU-baseline leg may import it; the product path never does.
"""
from .attention import (  # noqa: F401
    visibility,
    group_forward,
    group_backward,
    attention_forward,
    attention_backward,
    segments_from_cu_seqlens,
)
