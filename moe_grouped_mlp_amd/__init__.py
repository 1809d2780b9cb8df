"""Fused grouped-MLP MoE expert block for AMD Instinct MI355X (gfx950).

The compute path is the HIP library libmoe_gmlp.so (C ABI in
include/moe_gmlp.h); this package only marshals arguments to it.  PyTorch is
used for device memory and streams.  There is no fallback: if the library is
missing or fails to load, every call raises.
"""

from .binding import (  # noqa: F401
    ACT_GEGLU, ACT_SRELU, ACT_SWIGLU, DEVERR_DUP_EXPERT, DEVERR_MCAP_OVERFLOW,
    ERR_DEVICE, ERR_INVALID_ARG, ERR_LAUNCH, ERR_UNSUPPORTED, ERR_WORKSPACE,
    GROUP_ALIGN, INTERLEAVE, MX_BLOCK,
    PERMUTE_BUILD_MAP, PERMUTE_GATHER, PERMUTE_WRITE_MX, PERMUTE_WRITE_MX4, PREC_BF16,
    PREC_MXFP4, PREC_MXFP8, QUANT_BOTH, QUANT_COL, QUANT_ROW, MoeError, act_params, lib, lib_path,
    DEVERR_SYNC_TIMEOUT, DEVERR_BAD_OFFSETS, NOALLOC_SCRATCH_BYTES,
    moe_grouped_mlp_bwd, moe_grouped_mlp_bwd_noalloc, moe_grouped_mlp_fwd,
    moe_grouped_mlp_wgrad, moe_router_topk, moe_router_route,
    moe_router_route_workspace_size, moe_grouped_gemm, moe_glu_unfused,
    moe_grouped_mlp_workspace_size, moe_clock_tick_rate_hz,
    moe_gemm_clock_trace, CLOCK_MAX_WORKGROUPS, moe_bench_occupy,
    moe_grouped_gemm_workspace_size,
    moe_permute, moe_permute_workspace_size, moe_quantize_mxfp4, moe_quantize_mxfp8,
    moe_unpermute, moe_weight_repack_interleave, EXPORTED_SYMBOLS,
)
from .block import ExpertBlock  # noqa: F401
