// Un-permute and weighted combine with a fixed reduction order.
//
// "Expert outputs are combined with the normalised router weights, scaled by
// 2.5" (Reflection Beam 1.0 overview, section "Mixture of Experts"; the 2.5 is
// already inside the weights).  out[t] = bf16( sum_k w[t,k] * y[row(t,k)] ),
// summed in fp32 slot by slot (ascending expert id), each product rounded
// before the add, so the result does not depend on scheduling.
#include "common.h"

namespace beam {

// grid (T, ceil(H / 1024)); each thread owns 8 consecutive columns.  A token's K slot rows are
// loaded together, then added in slot order.
__global__ __launch_bounds__(128) void combine_kernel(int H, int K, const uint16_t* __restrict__ y,
                                                     const float* __restrict__ w,
                                                     const int32_t* __restrict__ pair_to_row,
                                                     uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int n = (blockIdx.y * 128 + threadIdx.x) * 8;
  if (n >= H) return;
  u32x4 v[kMaxTopK];
  float wk[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k < K) {
      const int p = t * K + k;
      wk[k] = w[p];
      v[k] = *reinterpret_cast<const u32x4*>(y + (size_t)pair_to_row[p] * H + n);
    }
  }
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k < K) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = __fadd_rn(acc[2 * j], __fmul_rn(wk[k], __uint_as_float(v[k][j] << 16)));
        acc[2 * j + 1] = __fadd_rn(acc[2 * j + 1], __fmul_rn(wk[k], __uint_as_float(v[k][j] & 0xFFFF0000u)));
      }
    }
  }
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = static_cast<uint32_t>(f32_to_bf16(acc[2 * j])) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * j + 1])) << 16);
  *reinterpret_cast<u32x4*>(out + (size_t)t * H + n) = o;
}

hipError_t launch_combine(const Shape& s, int T, const uint16_t* y, const float* w, const int32_t* pair_to_row,
                          uint16_t* out, hipStream_t stream) {
  if (s.K > kMaxTopK) return hipErrorInvalidValue;
  dim3 grid(T, (s.H + 1023) / 1024);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(128), 0, stream, s.H, s.K, y, w, pair_to_row, out);
  return hipGetLastError();
}

}  // namespace beam
