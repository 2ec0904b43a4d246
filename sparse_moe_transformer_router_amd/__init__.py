"""MI355X (gfx950) top-k routed MoE feed-forward layer with MXFP4 expert weights.

The compute lives in libmoe_mxfp4.so (hand-written HIP kernels behind a C ABI, declared in
include/moe_mxfp4.h); this package only loads it and marshals torch tensors into it.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    MOE_DTYPE_BF16,
    MOE_DTYPE_F32,
    MOE_FLAG_EMIT_ACT,
    MOE_FLAG_EMIT_PREACT,
    MOE_LAYOUT_ROWMAJOR,
    MOE_LAYOUT_TILED,
    MOE_PATH_AUTO,
    MOE_PATH_DECODE,
    MOE_PATH_DECODE_FUSED,
    MOE_PATH_GEMM,
    MOE_PATH_GEMM_MX,
    MOE_PATH_PREFILL_BF16,
    MOE_PATH_PREFILL_MX6SPLIT,
    MOE_PATH_PREFILL_MX8SPLIT,
    MOE_PATH_STREAM,
    MoeError,
    lib,
)
from .ops import (  # noqa: F401
    MXFP4Weight,
    Options,
    Router,
    abi_version,
    moe_attn_decode,
    moe_block_forward_ex,
    moe_combine,
    moe_forward,
    moe_forward_ex,
    moe_forward_noalloc,
    moe_mxfp4_dequant,
    moe_mxfp4_ffn,
    moe_mxfp4_pack,
    moe_mxfp4_tiled_bytes,
    moe_permute,
    moe_release_workspace,
    moe_rmsnorm,
    moe_route,
    moe_workspace_size,
    workspace,
)
