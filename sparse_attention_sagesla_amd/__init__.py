"""SageSLA attention forward for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libsagesla.so`` built from hand-written HIP
kernels (``csrc/``, interface in ``include/sagesla.h``); this package only marshals torch
tensors into it. The library is loaded on first use; there is no CPU fallback.
"""
from . import synth  # noqa: F401  (seeded synthetic inputs)
from ._lib import (GROUP, SageSLAError, adaptive_ksel, adaptive_workspace_layout,  # noqa: F401
                   adaptive_workspace_size, adaptive_workspace_views, alloc_workspace, fwd, fwd_adaptive,
                   fwd_prepared, ksel, lib, prepare,
                   sla_bwd, sla_fwd,
                   sla_workspace_layout, sla_workspace_size, sla_workspace_views, status_string,
                   w8a8_gemm, w8a8_linear, w8a8_quant_act, w8a8_quant_weight, w8a8_sizes, workspace_layout,
                   workspace_size, workspace_views)

__all__ = ["fwd", "ksel", "workspace_size", "workspace_layout", "workspace_views", "alloc_workspace",
           "SageSLAError", "status_string", "lib", "synth", "w8a8_sizes", "w8a8_quant_weight", "w8a8_quant_act",
           "w8a8_gemm", "w8a8_linear", "sla_fwd", "sla_bwd", "sla_workspace_size", "sla_workspace_layout",
           "sla_workspace_views", "prepare", "fwd_prepared", "fwd_adaptive", "adaptive_ksel",
           "adaptive_workspace_size", "adaptive_workspace_layout", "adaptive_workspace_views"]
