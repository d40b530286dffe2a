"""One DWDP rank's MoE hot path on AMD Instinct MI355X (gfx950).

The compute lives in libdwdp.so (hand-written HIP, C ABI in include/dwdp.h);
this package is its Python binding.  Importing it loads the library and fails
loudly if it has not been built: there is no other execution path.
"""
from . import _lib

_lib.load()

from . import api  # noqa: E402,F401
from .moe import DWDPPipeline, ExpertStore, LayerWeights, MoEBlock, dwdp_placement  # noqa: E402,F401

__all__ = ["api", "DWDPPipeline", "ExpertStore", "LayerWeights", "MoEBlock", "dwdp_placement"]
