"""Beam MoE block forward pass on MI355X (gfx950): HIP kernels behind a C ABI.

The layer: sigmoid router over all experts, group-limited top-k (groups ranked
by the sum of their top-2 scores), normalised weights scaled by alpha, SwiGLU
experts, weighted combine (Reflection Beam 1.0 overview page, section
"Mixture of Experts").  The functions below marshal torch tensors into the
C ABI of libbeam_moe.so (include/beam_moe.h); every step runs in HIP kernels.
"""
from .binding import (  # noqa: F401
    BeamMoeError,
    Config,
    DenseConfig,
    LAYOUT_FRAGMENTS,
    LAYOUT_ROWS,
    LIB_PATH,
    MAX_NORM_HIDDEN,
    MAX_TOKENS,
    OP_BLOCK,
    OP_FORWARD,
    OP_PERMUTE,
    OP_ROUTE,
    W_BF16,
    W_FP8_E4M3,
    W_MXFP4,
    beam_dense_mlp_forward,
    beam_dense_workspace_bytes,
    beam_moe_block_forward,
    beam_moe_forward,
    beam_moe_forward_noalloc,
    NOALLOC_SCRATCH_BYTES,
    beam_moe_pack_scales,
    beam_moe_pack_weights,
    beam_moe_permute,
    beam_moe_rms_norm,
    beam_moe_route,
    beam_moe_workspace_bytes,
    beam_mxfp4_quantize,
    status_string,
)
