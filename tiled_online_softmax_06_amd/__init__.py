"""FlashAttention forward for MI355X (gfx950): exact softmax(scale * Q K^T) V
computed tile by tile with a running row max and normaliser.

``forward`` and ``forward_into`` are thin ctypes bindings of the C-ABI
library ``libfa.so`` (see include/fa.h); every step of the computation runs
in its HIP kernels.  ``inputs`` builds the seeded synthetic workloads.
"""
from .fa import (  # noqa: F401
    backward,
    backward_into,
    forward,
    forward_fp8,
    forward_fp8_into,
    forward_into,
    forward_split,
    forward_split_into,
    library_path,
    load_library,
    merge,
    merge_into,
    split_suggest,
    split_workspace_bytes,
)
