"""CPU oracle for the Beam MoE layer forward pass (test infrastructure only).

This package is test infrastructure.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path (the HIP library
and its Python binding) never does, and it shares no code with that path.

Every function here is the plain definition of a step of the layer, written
in NumPy with fp64 accumulation and rounding to fp32/bf16 at the points the
layer fixes.  See oracle/moe.py for the step-by-step citations.

Parity status of each function:
  codecs.bf16_round_bits / bf16_to_f64 / e4m3_decode  -- pinned (library casts, all codes)
  codecs.e2m1_decode / mxfp4_unpack / mxfp4_dequant /  -- pinned (torch's own e2m1 conversions:
  mxfp4_quantize / e8m0_scale                             codes, element rounding, packing; the
                                                          shared-exponent rule; on-grid round
                                                          trips; the error bound, saturation and
                                                          zero blocks; planted mutants caught)
  moe.router_scores / select_experts / route          -- pinned (brute force, invariants,
                                                          the G=1 plain top-k special case)
  moe.permute                                          -- pinned (stable argsort, invariants)
  moe.expert_rows / forward                            -- pinned (naive loops, identical-
                                                          experts special case, dense-MLP
                                                          reduction)
  moe.forward at the real shape                        -- values are the definition; the
                                                          pages print no worked example
  block.rms_norm_bits / mix_weights / residual_mix_bits -- pinned (exact-sum bound, closed
                                                          forms, unit-scale invariants)
  block.block_forward                                  -- composition of pinned steps
  moe.dense_mlp                                        -- pinned (naive loops; equals the
                                                          MoE layer with identical experts / 2.5)
"""
from . import block, codecs, moe  # noqa: F401
from .moe import (  # noqa: F401
    LayerSpec,
    router_logits,
    router_scores,
    select_experts,
    combine_weights,
    route,
    gap_violations,
    permute,
    expert_rows,
    combine,
    dense_mlp,
    forward,
)
from .block import block_forward, mix_weights, residual_mix_bits, rms_norm_bits  # noqa: F401
