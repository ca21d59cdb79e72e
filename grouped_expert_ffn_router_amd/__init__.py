"""MI355X-native fixed-pool, three-wave MoE expert layer (one EP rank).

The layer runs in libmoe.so (hand-written HIP kernels for gfx950 behind the C
ABI of include/moe.h).  ``binding`` marshals arguments into that ABI and
``runner`` lays out device buffers with torch; neither computes any part of
the layer.
"""

from . import binding  # noqa: F401

__all__ = ["binding"]
