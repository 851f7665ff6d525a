"""W4A16 mixture-of-experts grouped GEMM for AMD MI355X (gfx950).

The computation lives in ``libw4a16.so`` (HIP kernels behind the C ABI of
``include/w4a16.h``); this package only builds and binds it.
"""
from .lib import (FORMAT_INT4, FORMAT_MXFP4, FUSED_STAGE_EVENTS, FUSED_STAGES, KERNEL_DECODE,  # noqa: F401
                  KERNEL_PREFILL, Plan, W4A16Error,
                  Weights, contiguous_workspace_bytes, dequant, fused_moe, fused_moe_plans, fused_moe_workspace_bytes,
                  gemm_workspace_bytes, grouped_gemm, grouped_gemm_contiguous, grouped_gemm_masked,
                  grouped_gemm_offsets, grouped_gemm_silu, load, make_plan, masked_workspace_bytes, moe_combine,
                  pack_weights, pack_weights_mxfp4,
                  packed_bytes, plan_select, route_bounds, route_prep, route_prep_into, route_prep_workspace_bytes,
                  silu_mul, validate_routing, version, zeroed_workspace)
