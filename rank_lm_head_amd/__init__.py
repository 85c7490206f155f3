"""MI355X-native low-rank draft LM head (EAGLE-4's cheap candidate head).

The compute lives in liblrhead.so (hand-written HIP kernels for gfx950 behind
the C ABI of include/lrhead.h); this package is its thin Python binding.
"""
from ._lib import BF16, FP32, LrheadError, load  # noqa: F401
from .head import Head, branch, draft_static, factor  # noqa: F401

__all__ = ["Head", "branch", "draft_static", "factor", "LrheadError", "load", "BF16", "FP32"]
