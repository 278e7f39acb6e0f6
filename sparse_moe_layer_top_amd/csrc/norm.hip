// RMSNorm before the MoE block, and the post-norm + constant-scale residual mix
// fused into the combine.
//
// Reflection Beam 1.0 overview, section "Residual stream": every sublayer is
// normalised before and after, the norms in FP32; the embedding is step 1 and
// at step k the sublayer output joins the stream with weight 1/sqrt(k) while
// the stream keeps sqrt((k-1)/k).  The norm is RMSNorm with a per-channel gain:
//   n = v / sqrt(mean(v^2) + eps),  out = bf16(n * gamma),
// every step one correctly rounded FP32 operation, the sum of squares taken over
// the channels in index order; the mix is
//   new = bf16( fp32(a * stream) + fp32(b * post) ),  a = sqrt((k-1)/k), b = 1/sqrt(k),
// with a and b rounded once to FP32 on the host.  Both kernels use one wave per
// token: the row is staged in LDS, lane 0 runs the sequential sum (the chain the
// definition fixes), and the whole wave applies the scale.
#include "common.h"
#include "rn_math.h"

namespace beam {

// Sequential fp32 sum of squares of a bf16 row in LDS (channel order).
__device__ __forceinline__ float row_sumsq(const uint16_t* row, int H) {
  float ss = 0.f;
  for (int c = 0; c < H; c += 8) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __uint_as_float(v[j] << 16), hi = __uint_as_float(v[j] & 0xFFFF0000u);
      ss = __fadd_rn(ss, __fmul_rn(lo, lo));
      ss = __fadd_rn(ss, __fmul_rn(hi, hi));
    }
  }
  return ss;
}

// r = 1 / sqrt(ss / H + eps), each step correctly rounded.
__device__ __forceinline__ float rms_scale(float ss, int H, float eps) {
  const float ms = __fdiv_rn(ss, static_cast<float>(H));
  return __fdiv_rn(1.0f, sqrt_rn(__fadd_rn(ms, eps)));
}

// bf16((v * r) * gamma) on 8 packed bf16 values
__device__ __forceinline__ u32x4 scale_gain8(u32x4 v, float r, const float* g) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = __fmul_rn(__fmul_rn(__uint_as_float(v[j] << 16), r), g[2 * j]);
    const float hi = __fmul_rn(__fmul_rn(__uint_as_float(v[j] & 0xFFFF0000u), r), g[2 * j + 1]);
    o[j] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
  }
  return o;
}

// grid T, block 64, dynamic LDS H*2 bytes.  out may alias in: the row is staged
// in LDS before anything is written.
__global__ __launch_bounds__(64) void rms_norm_kernel(int H, float eps, const uint16_t* in,
                                                      const float* __restrict__ gamma, uint16_t* out) {
  extern __shared__ __attribute__((aligned(16))) uint16_t row[];
  __shared__ float s_r;
  const int t = blockIdx.x, lane = threadIdx.x;
  const uint16_t* src = in + (size_t)t * H;
  for (int c = lane * 8; c < H; c += 64 * 8) *reinterpret_cast<u32x4*>(row + c) = *reinterpret_cast<const u32x4*>(src + c);
  __syncthreads();
  if (lane == 0) s_r = rms_scale(row_sumsq(row, H), H, eps);
  __syncthreads();
  const float r = s_r;
  uint16_t* dst = out + (size_t)t * H;
  for (int c = lane * 8; c < H; c += 64 * 8) {
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = gamma[c + j];
    *reinterpret_cast<u32x4*>(dst + c) = scale_gain8(*reinterpret_cast<const u32x4*>(row + c), r, g);
  }
}

// Combine (as combine_kernel: fixed slot order, unfused mul/add) of token t into
// LDS (and moe_out if given), then post-norm and the residual mix into stream_out.
// grid T, block 64, dynamic LDS H*2 bytes.  stream_out may alias stream_in: each
// lane reads its chunk of the stream before writing that chunk.
__global__ __launch_bounds__(64) void combine_norm_mix_kernel(int H, int K, const uint16_t* __restrict__ y,
                                                              const float* __restrict__ w,
                                                              const int32_t* __restrict__ pair_to_row,
                                                              float eps, const float* __restrict__ gamma, float a,
                                                              float b, const uint16_t* stream_in,
                                                              uint16_t* stream_out, uint16_t* __restrict__ moe_out) {
  extern __shared__ __attribute__((aligned(16))) uint16_t row[];
  __shared__ float s_r;
  const int t = blockIdx.x, lane = threadIdx.x;
  for (int c = lane * 8; c < H; c += 64 * 8) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int p = t * K + k;
      const float wk = w[p];
      const u32x4 v = *reinterpret_cast<const u32x4*>(y + (size_t)pair_to_row[p] * H + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = __fadd_rn(acc[2 * j], __fmul_rn(wk, __uint_as_float(v[j] << 16)));
        acc[2 * j + 1] = __fadd_rn(acc[2 * j + 1], __fmul_rn(wk, __uint_as_float(v[j] & 0xFFFF0000u)));
      }
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = static_cast<uint32_t>(f32_to_bf16(acc[2 * j])) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * j + 1])) << 16);
    *reinterpret_cast<u32x4*>(row + c) = o;
    if (moe_out) *reinterpret_cast<u32x4*>(moe_out + (size_t)t * H + c) = o;
  }
  __syncthreads();
  if (lane == 0) s_r = rms_scale(row_sumsq(row, H), H, eps);
  __syncthreads();
  const float r = s_r;
  for (int c = lane * 8; c < H; c += 64 * 8) {
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = gamma[c + j];
    const u32x4 p = scale_gain8(*reinterpret_cast<const u32x4*>(row + c), r, g);
    const u32x4 s = *reinterpret_cast<const u32x4*>(stream_in + (size_t)t * H + c);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __fadd_rn(__fmul_rn(a, __uint_as_float(s[j] << 16)), __fmul_rn(b, __uint_as_float(p[j] << 16)));
      const float hi = __fadd_rn(__fmul_rn(a, __uint_as_float(s[j] & 0xFFFF0000u)),
                                 __fmul_rn(b, __uint_as_float(p[j] & 0xFFFF0000u)));
      o[j] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
    }
    *reinterpret_cast<u32x4*>(stream_out + (size_t)t * H + c) = o;
  }
}

hipError_t launch_rms_norm(int T, int H, float eps, const uint16_t* in, const float* gamma, uint16_t* out,
                           hipStream_t stream) {
  hipLaunchKernelGGL(rms_norm_kernel, dim3(T), dim3(64), (size_t)H * 2, stream, H, eps, in, gamma, out);
  return hipGetLastError();
}

hipError_t launch_combine_norm_mix(const Shape& s, int T, const uint16_t* y, const float* w, const int32_t* pair_to_row,
                                   float eps, const float* gamma, float a, float b, const uint16_t* stream_in,
                                   uint16_t* stream_out, uint16_t* moe_out, hipStream_t stream) {
  hipLaunchKernelGGL(combine_norm_mix_kernel, dim3(T), dim3(64), (size_t)s.H * 2, stream, s.H, s.K, y, w, pair_to_row,
                     eps, gamma, a, b, stream_in, stream_out, moe_out);
  return hipGetLastError();
}

}  // namespace beam
