"""MI355X-native (gfx950) Gated DeltaNet-2 chunkwise operator.

``fwd`` and ``bwd`` are thin ctypes wrappers over ``libgdn2.so`` (C ABI in
``include/gdn2.h``); all arithmetic runs in its HIP kernels.  Build the library
with ``python -m linear_attention_sequence_gdn2_amd.build``.
"""
from ._binding import (EXPORTS, LIB_PATH, Gdn2Error, Gdn2Shape, bwd, bwd_workspace_bytes, fwd,  # noqa: F401
                       load, make_shape)

__all__ = ["fwd", "bwd", "load", "bwd_workspace_bytes", "Gdn2Error", "Gdn2Shape", "LIB_PATH", "EXPORTS",
           "make_shape"]
