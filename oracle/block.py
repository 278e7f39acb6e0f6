"""Plain CPU definition of the norms and the residual mix around the MoE block
(test infrastructure only).

What the pages state (Reflection Beam 1.0 overview, agentlenshq.com, section
"Residual stream: ..."; the same facts on the aixai.ru page, section "Residual
stream with constant scale", and on the dothoosh.com page, section on the
residual stream):

  * the input embedding counts as step 1; at step k a sublayer's output is added
    with weight 1/sqrt(k) while the running stream keeps weight sqrt((k-1)/k),
    so the two squared weights sum to one and the stream keeps its scale;
  * every sublayer is normalised both before and after;
  * the implementation computes the norms in FP32 (with the router, the SwiGLU
    product, RoPE, query scaling and the logit soft-cap).

Readings this module takes where the pages are silent:
  * the norm is RMSNorm with a learned per-channel gain (the only norm the pages
    name, on queries and keys) and an additive epsilon inside the square root:
        n = v / sqrt(mean(v^2) + eps),  out = n * gamma;
  * "in FP32" is taken literally, one IEEE float32 result per step: the sum
    of squares is the exact sum rounded once to float32 (the pages fix the
    precision, not an order of additions, so the definition takes none), then
    one correctly rounded division by H, one addition of eps, one correctly
    rounded square root and one reciprocal; then v * r, then * gamma;
  * the stream, the MoE output and both norm outputs are bf16 (the model dtype),
    each norm output rounded once to nearest-even;
  * the mix is new = bf16( f32(a * stream) + f32(b * post) ) with the weights
    a = sqrt((k-1)/k) and b = 1/sqrt(k) rounded once from float64 to float32.

Every value here is float32 or bf16; float32 products of bf16 values are exact
(8-bit significands), so the only roundings are the ones listed.
"""
from __future__ import annotations

import math
from typing import Callable

import numpy as np

from .codecs import bf16_round_bits, bf16_to_f64
from .moe import LayerSpec, forward


def _round_f32_exact(sq: np.ndarray) -> np.float32:
    """The exact sum of the float64 values sq (each exact), rounded once to float32 (nearest, ties to even).

    math.fsum returns the exact sum rounded to float64.  Rounding that to
    float32 can round twice only when it lands exactly halfway between two
    float32 values; then the sign of the exact remainder (fsum of the terms
    minus that midpoint, whose sign fsum gets right) decides the direction.
    """
    s64 = math.fsum(sq)
    r = np.float32(s64)
    if not np.isfinite(r) or float(r) == s64:
        return r
    other = np.nextafter(r, np.float32(np.inf) if float(r) < s64 else np.float32(-np.inf))
    if s64 - float(r) != float(other) - s64:            # not a float32 midpoint: one rounding
        return r
    rem = math.fsum(list(sq) + [-s64])                   # exact sum minus the midpoint, sign exact
    if rem == 0.0:
        return r                                         # a true tie: numpy already chose the even one
    up = rem > 0.0
    lo, hi = (r, other) if float(r) < float(other) else (other, r)
    return hi if up else lo


def sum_squares_f32(v) -> np.ndarray:
    """float32 sum of squares of float32 rows [T, H]: the exact sum, rounded once.

    The rows are bf16 values, so each square is exact in float64 (16 significant
    bits), and the float32 result does not depend on an order of additions.
    """
    v = np.asarray(v, np.float32)
    sq = v.astype(np.float64) ** 2
    return np.array([_round_f32_exact(row) for row in sq], np.float32)


def rms_norm_bits(v_bits, gamma, eps: float) -> np.ndarray:
    """RMSNorm of bf16 rows [T, H] with float32 gain gamma [H] -> bf16 bits [T, H].

    Sum of squares: the exact sum rounded once to float32 (sum_squares_f32);
    then ms = ss / H,
    r = 1 / sqrt(ms + eps), out = bf16((v * r) * gamma), each step one float32
    operation.
    """
    v = bf16_to_f64(np.asarray(v_bits, np.uint16)).astype(np.float32)
    if v.ndim == 1:
        v = v[None, :]
    T, H = v.shape
    g = np.asarray(gamma, np.float32)
    ss = sum_squares_f32(v)
    ms = ss / np.float32(H)
    r = np.float32(1.0) / np.sqrt(ms + np.float32(eps))
    n = v * r[:, None]
    return bf16_round_bits(n * g[None, :])


def mix_weights(step: int):
    """(a, b) = (sqrt((k-1)/k), 1/sqrt(k)) for step k >= 2, each rounded once to float32."""
    if step < 2:
        raise ValueError("a sublayer's step k is at least 2 (the embedding is step 1)")
    return np.float32(math.sqrt((step - 1) / step)), np.float32(1.0 / math.sqrt(step))


def residual_mix_bits(stream_bits, post_bits, step: int) -> np.ndarray:
    """new = bf16( f32(a * stream) + f32(b * post) ), a = sqrt((k-1)/k), b = 1/sqrt(k)."""
    a, b = mix_weights(step)
    s = bf16_to_f64(np.asarray(stream_bits, np.uint16)).astype(np.float32)
    p = bf16_to_f64(np.asarray(post_bits, np.uint16)).astype(np.float32)
    return bf16_round_bits(a * s + b * p)


def block_forward(spec: LayerSpec, stream_bits, gamma_pre, gamma_post, eps: float, step: int,
                  w_router, b_router, weights: Callable[[str, int], object]):
    """Pre-norm -> MoE block -> post-norm -> constant-scale residual mix.

    Returns the MoE dict of oracle.moe.forward (computed on the normalised input)
    plus x (the pre-norm output, the block's input), post (the post-norm output)
    and stream_out.
    """
    stream_bits = np.asarray(stream_bits, np.uint16)
    x = rms_norm_bits(stream_bits, gamma_pre, eps)
    res = forward(spec, x, w_router, b_router, weights)
    post = rms_norm_bits(res["out"], gamma_post, eps)
    res.update(x=x, post=post, stream_out=residual_mix_bits(stream_bits, post, step))
    return res
