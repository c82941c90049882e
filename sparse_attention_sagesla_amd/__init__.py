"""SageSLA attention forward for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libsagesla.so`` built from hand-written HIP
kernels (``csrc/``); this package only marshals torch tensors into it. The library
is loaded on first use; there is no CPU fallback.
"""
from . import synth  # noqa: F401  (seeded synthetic inputs)

__all__ = ["synth"]
