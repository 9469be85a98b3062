"""MI355X (gfx950) MoE sublayer forward with FarSkip-Collective wiring.

The compute lives in libfarskip_moe.so (hand-written HIP kernels behind the C ABI of
include/farskip_moe.h); this package only loads it and marshals torch tensors into it.
"""
from ._lib import LIB_PATH, EXPORTS, FarSkipMoEError, lib  # noqa: F401
from . import ops  # noqa: F401

__all__ = ["lib", "ops", "FarSkipMoEError", "LIB_PATH", "EXPORTS"]
