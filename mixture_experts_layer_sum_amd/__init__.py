"""MI355X (gfx950) MoE sublayer forward with FarSkip-Collective wiring.

The compute lives in libfarskip_moe.so (hand-written HIP kernels behind the C ABI of
include/farskip_moe.h); this package only loads it and marshals torch tensors into it.  The library
is loaded on first use of `lib` or `ops` (importing `mixture_experts_layer_sum_amd.build` does not
need it); a missing library raises ImportError there, there is no fallback.
"""
import importlib

__all__ = ["lib", "ops", "FarSkipMoEError", "LIB_PATH", "EXPORTS"]


def __getattr__(name):
    if name in ("lib", "FarSkipMoEError", "LIB_PATH", "EXPORTS"):
        return getattr(importlib.import_module("._lib", __name__), name)
    if name == "ops":
        return importlib.import_module(".ops", __name__)
    raise AttributeError(name)
