"""Single-GPU sparse MoE layer forward for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library libmoe_mi355x.so (C ABI in include/moe.h);
this package is its ctypes binding plus a layer runner that owns the device
buffers.  Importing the package does not load the library; the first call does,
and fails loudly when the library has not been built.
"""
from ._lib import (MOE_BF16, MOE_F32, MOE_SIGMOID, MOE_SOFTMAX, MoeBiasStats, MoeError,
                   load, moe_bias_update, moe_combine, moe_grouped_swiglu,
                   moe_grouped_swiglu_workspace_size, moe_last_error, moe_permute,
                   moe_permute_workspace_size, moe_profile_enable, moe_profile_only, moe_profile_report,
                   moe_profile_tag,
                   moe_route, moe_route_workspace_size,
                   moe_version)
from .layer import LayerShape, MoELayer

__all__ = ["MOE_BF16", "MOE_F32", "MOE_SIGMOID", "MOE_SOFTMAX", "MoeBiasStats", "MoeError",
           "load", "moe_bias_update", "moe_combine", "moe_grouped_swiglu",
           "moe_grouped_swiglu_workspace_size", "moe_last_error", "moe_permute",
           "moe_permute_workspace_size", "moe_profile_enable", "moe_profile_only", "moe_profile_report",
           "moe_profile_tag", "moe_route", "moe_route_workspace_size",
           "moe_version", "LayerShape", "MoELayer"]
