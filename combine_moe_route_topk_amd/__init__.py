"""MI355X (gfx950) MoE routing, dispatch and combine.

The compute lives in the HIP library ``libmoe_dc.so`` (C ABI in
``include/moe_dc.h``); this package is its PyTorch binding.  Importing it
without the built library raises ImportError -- there is no CPU fallback.
"""
from .api import (DispatchResult, MoeError, default_sort_cutoff, moe_abi_version, moe_combine, moe_dequant_rows,
                  moe_dispatch, moe_dispatch_workspace_bytes, moe_gather_rows,
                  moe_gather_swiglu, moe_gather_swiglu_combine,
                  moe_gather_swiglu_workspace_bytes,
                  moe_grouped_gemm_fp8, moe_grouped_swiglu,
                  moe_grouped_swiglu_workspace_bytes, moe_resolve_sorted, moe_route_dispatch,
                  moe_route_dispatch_noalloc, moe_route_dispatch_workspace_bytes, moe_route_topk,
                  moe_scatter_rows)
from ._lib import LIB_PATH, MOE_NOALLOC_SCRATCH_BYTES, MOE_SORT_AUTO, MOE_SORT_OFF, MOE_SORT_ON

__all__ = ["DispatchResult", "MoeError", "default_sort_cutoff", "moe_abi_version", "moe_combine", "moe_dequant_rows",
           "moe_dispatch", "moe_dispatch_workspace_bytes", "moe_gather_rows",
           "moe_gather_swiglu", "moe_gather_swiglu_combine",
           "moe_gather_swiglu_workspace_bytes",
           "moe_grouped_gemm_fp8", "moe_grouped_swiglu",
           "moe_grouped_swiglu_workspace_bytes", "moe_resolve_sorted", "moe_route_topk",
           "moe_scatter_rows", "moe_route_dispatch", "moe_route_dispatch_noalloc",
           "moe_route_dispatch_workspace_bytes",
           "LIB_PATH", "MOE_NOALLOC_SCRATCH_BYTES", "MOE_SORT_AUTO", "MOE_SORT_OFF", "MOE_SORT_ON"]
