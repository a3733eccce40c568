"""MI355X (gfx950) exact attention: FlashAttention-2 forward and backward as HIP kernels.

``forward`` / ``backward`` call libfa2.so (C ABI in include/fa2.h) through a
thin ctypes binding; ``inputs`` and ``workloads`` hold the seeded synthetic
inputs and the benchmark shapes.
"""
from .fa2 import FA2Error, backward, forward, workspace_bytes  # noqa: F401
