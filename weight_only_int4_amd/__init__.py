"""W4A16 mixture-of-experts grouped GEMM for AMD MI355X (gfx950).

The computation lives in ``libw4a16.so`` (HIP kernels behind the C ABI of
``include/w4a16.h``); this package only builds and binds it.
"""
from .lib import (KERNEL_DECODE, KERNEL_PREFILL, Plan, W4A16Error, Weights, dequant, fused_moe,  # noqa: F401
                  fused_moe_plans, fused_moe_workspace_bytes, gemm_workspace_bytes, grouped_gemm, grouped_gemm_offsets, load, make_plan, moe_combine,
                  pack_weights, packed_bytes, plan_select, route_bounds, route_prep, route_prep_into, silu_mul, zeroed_workspace,
                  version)
