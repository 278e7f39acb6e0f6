// Correctly rounded float32 square root, usable on the host and the device.
//
// The norms around the MoE block are computed in FP32 (Reflection Beam 1.0
// overview, section "Residual stream"); for their results to be reproducible
// bit for bit, each FP32 step must be correctly rounded.  v_sqrt_f32 is not
// (its error bound is an ulp), so the root is settled from the definition of
// rounding to nearest:
//
//   s = fp32(sqrt(fp64(x)))    is within an ulp of the root;
//   m- = (s + prev(s)) / 2,  m+ = (s + next(s)) / 2    (exact in fp64)
//   the correctly rounded root is prev(s) if x < m-^2, next(s) if x > m+^2,
//   else s.  m-^2 and m+^2 are exact in fp64: m has at most 25 significant
//   bits.  x never equals a midpoint's square (that would need 50 bits).
//
// Valid for finite x > 0 whose root is a normal float (x >= 2^-252 suffices);
// the callers pass mean(v^2) + eps with eps > 0.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define BEAM_RN_FN __host__ __device__ __forceinline__
#else
#define BEAM_RN_FN static inline
#endif

namespace beam {

BEAM_RN_FN float sqrt_rn(float x) {
  const double xd = static_cast<double>(x);
  float s = static_cast<float>(__builtin_sqrt(xd));
  const uint32_t u = __builtin_bit_cast(uint32_t, s);
  const float below = __builtin_bit_cast(float, u - 1u);
  const float above = __builtin_bit_cast(float, u + 1u);
  const double lo = (static_cast<double>(s) + static_cast<double>(below)) * 0.5;
  const double hi = (static_cast<double>(s) + static_cast<double>(above)) * 0.5;
  if (xd < lo * lo) {
    s = below;
  } else if (xd > hi * hi) {
    s = above;
  }
  return s;
}

}  // namespace beam
