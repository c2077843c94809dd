"""Fused Mixture-of-Experts layer for one AMD MI355X (gfx950).

The layer -- top-k softmax router, expert-sorted token permutation, grouped
expert GEMMs with a fused SiLU*up epilogue, weighted un-permute combine --
runs in hand-written HIP kernels behind the C ABI of include/moe.h
(libmoe.so); this package is its thin ctypes binding plus the seeded input
generator used by tests and benchmarks.
"""
from ._binding import (MOE_BF16, FusedForwardGraph, MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED,
                       MOE_ERR_WORKSPACE, MOE_FP8_E4M3, MOE_FP8_E4M3_ROWWISE, MOE_MXFP4_E2M1, MOE_OK, MOE_REGIME_AUTO,
                       MOE_REGIME_DECODE, MOE_REGIME_PREFILL, MoEError, NOALLOC_SCRATCH_BYTES, Plan, fused_plan, fused_routing, load_library,
                       moe_align, moe_align_ex, moe_fused_forward, moe_fused_forward_noalloc,
                       moe_quant_rows_e4m3, moe_topk,
                       status_string, workspace_size)

__all__ = [
    "MOE_BF16", "MOE_FP8_E4M3", "MOE_FP8_E4M3_ROWWISE", "MOE_MXFP4_E2M1", "MOE_OK", "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED",
    "MOE_ERR_WORKSPACE", "MOE_ERR_HIP", "MOE_REGIME_AUTO", "MOE_REGIME_DECODE",
    "MOE_REGIME_PREFILL", "MoEError", "load_library", "moe_topk", "moe_align", "moe_align_ex",
    "moe_quant_rows_e4m3", "moe_fused_forward", "status_string", "workspace_size",
    "FusedForwardGraph", "Plan", "fused_plan", "fused_routing", "moe_fused_forward_noalloc",
    "NOALLOC_SCRATCH_BYTES",
]
