"""MI355X-native single-step decode attention for Reference Sliding Window
Attention (R-SWA) and Sparse R-SWA (SR-SWA).

    from long_context_decode_attn_amd import uocr      # C-ABI binding
    from long_context_decode_attn_amd import synth     # seeded workloads
    from long_context_decode_attn_amd.session import DecodeSession

The compute lives in libuocr.so (hand-written gfx950 HIP kernels behind the C
ABI declared in include/uocr.h); build it with
`python -m long_context_decode_attn_amd.build`.
"""
from . import synth  # noqa: F401
from . import uocr  # noqa: F401

__all__ = ["synth", "uocr"]
