"""MI355X (gfx950) CARVE key-axis gated delta rule: HIP kernels behind a C ABI.

    from chunk_gated_delta_amd import fwd, bwd

`fwd` / `bwd` marshal torch tensors into the C ABI of libcarve.so; the
library is loaded on first use and must be built (chunk_gated_delta_amd.build).
"""
from .carve import fwd, bwd, fwd_save, bwd_saved, load_library, fwd_workspace_bytes  # noqa: F401

__all__ = ["fwd", "bwd", "fwd_save", "bwd_saved", "load_library", "fwd_workspace_bytes"]
