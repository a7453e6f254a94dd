"""MI355X-native (gfx950) Gated DeltaNet-2 chunkwise operator.

``fwd`` and ``bwd`` are thin ctypes wrappers over ``libgdn2.so`` (C ABI in
``include/gdn2.h``); all arithmetic runs in its HIP kernels.  Build the library
with ``python -m linear_attention_sequence_gdn2_amd.build``.
"""
from ._binding import (EXPORTS, LIB_PATH, Gdn2Error, Gdn2Shape, bwd, bwd_factors, bwd_grads,  # noqa: F401
                       bwd_reverse, bwd_saved, bwd_workspace_bytes, chunk_states, factors_bytes, fwd, fwd_factored,
                       fwd_noalloc, fwd_output, fwd_output_fused, fwd_output_xerr, fwd_states,
                       load, make_shape, output_bwd, output_bwd_workspace_bytes, output_fwd, states_shape,
                       step, sweeps, sweeps_fused)

__all__ = ["fwd", "bwd", "fwd_states", "chunk_states", "bwd_factors", "bwd_reverse", "bwd_grads", "bwd_saved",
           "load", "bwd_workspace_bytes", "factors_bytes", "states_shape", "Gdn2Error", "Gdn2Shape", "LIB_PATH",
           "EXPORTS", "make_shape", "step", "output_fwd", "output_bwd",
           "output_bwd_workspace_bytes", "fwd_factored", "sweeps", "sweeps_fused", "fwd_noalloc", "fwd_output",
           "fwd_output_fused", "fwd_output_xerr"]
