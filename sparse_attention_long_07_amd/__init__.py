"""Native Sparse Attention (NSA) forward and decode step for MI355X (gfx950).

The compute path is the C-ABI library ``libnsa.so`` (hand-written HIP
kernels); :mod:`.nsa` binds it.  PyTorch supplies device memory and streams.
"""
from .config import NSAShape, WORKLOADS  # noqa: F401
