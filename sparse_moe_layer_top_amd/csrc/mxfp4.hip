// MXFP4 quantisation of bf16 rows (the OCP Microscaling conversion rule; MXFP4
// is the MI355X analogue of the NVFP4 checkpoint on the Reflection Beam 1.0
// overview page, section "Mixture of Experts").
//
// Per block of 32 consecutive values: shared = floor(log2(max|v|)) - 2, clamped
// to [-127, 127]; scale byte = shared + 127 (0 for an all-zero block); each
// v / 2^shared (exact) is rounded to the nearest E2M1 magnitude
// {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating at 6; the
// sign code is set for v < 0.  Only integer and compare steps: bit-exact.
#include "common.h"

namespace beam {

// floor(log2(|v|)) of a nonzero finite bf16 magnitude (15 bits)
__device__ __forceinline__ int bf16_floor_log2(uint32_t mag) {
  const int e = static_cast<int>(mag >> 7);
  if (e > 0) return e - 127;
  return (31 - __clz(static_cast<int>(mag & 0x7Fu))) - 133;   // subnormal: m * 2^-133
}

// |v| / 2^shared (in [0, 8)) -> E2M1 magnitude code, nearest with ties to even, saturating
__device__ __forceinline__ uint32_t e2m1_round(float u) {
  const float mid[8] = {0.f, 0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  uint32_t c = 0;
#pragma unroll
  for (int k = 1; k < 8; ++k)
    if (u > mid[k] || (u == mid[k] && (k % 2 == 0))) c = static_cast<uint32_t>(k);
  return c;
}

// one thread per 32-value block: grid-stride over rows * cols/32 blocks
__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(int rows, int cols, const uint16_t* __restrict__ w,
                                                             uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const long nblk = (long)rows * (cols / 32);
  for (long b = (long)blockIdx.x * 256 + threadIdx.x; b < nblk; b += (long)gridDim.x * 256) {
    const uint16_t* src = w + b * 32;        // blocks are contiguous: row r, block k at (r * cols/32 + k) * 32
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const u32x4*>(src + 8 * i);
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) amax = max(amax, max(v[i][j] & 0x7FFFu, (v[i][j] >> 16) & 0x7FFFu));
    int shared = 0;
    uint32_t ebyte = 0;
    if (amax != 0) {
      shared = min(max(bf16_floor_log2(amax) - 2, -127), 127);
      ebyte = static_cast<uint32_t>(shared + 127);
    }
    u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t bits = h ? (v[i][j] >> 16) : (v[i][j] & 0xFFFFu);
          const uint32_t mag = bits & 0x7FFFu;
          const float u = amax ? ldexpf(__uint_as_float(mag << 16), -shared) : 0.f;
          const uint32_t code = e2m1_round(u) | ((bits & 0x8000u) && mag ? 8u : 0u);
          const int idx = 8 * i + 2 * j + h;                      // value index in the block
          out[idx / 8] |= code << (4 * (idx % 8));
        }
    *reinterpret_cast<u32x4*>(codes + b * 16) = out;
    scales[b] = static_cast<uint8_t>(ebyte);
  }
}

hipError_t launch_mxfp4_quantize(int rows, int cols, const uint16_t* w, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream) {
  const long nblk = (long)rows * (cols / 32);
  const int grid = (int)std::min<long>((nblk + 255) / 256, 16384);
  hipLaunchKernelGGL(mxfp4_quantize_kernel, dim3(grid), dim3(256), 0, stream, rows, cols, w, codes, scales);
  return hipGetLastError();
}

}  // namespace beam
