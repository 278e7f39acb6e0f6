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
// token: every lane squares its channels (exact in FP32) into LDS, lane 0 runs
// the sequential sum (the chain the definition fixes), and the whole wave
// applies the scale to the row it holds in registers.
#include "beam_moe.h"
#include "common.h"
#include "rn_math.h"

namespace beam {

constexpr int kNormMaxChunks = BEAM_MOE_MAX_NORM_HIDDEN / (64 * 8);   // 8-channel chunks per lane

// Squares of 8 packed bf16 values (exact in fp32: 8-bit significands) into sq[c .. c+7].
__device__ __forceinline__ void store_squares8(float* sq, int c, u32x4 v) {
  f32x4 a, b;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float l0 = __uint_as_float(v[j] << 16), h0 = __uint_as_float(v[j] & 0xFFFF0000u);
    const float l1 = __uint_as_float(v[j + 2] << 16), h1 = __uint_as_float(v[j + 2] & 0xFFFF0000u);
    a[2 * j] = __fmul_rn(l0, l0);
    a[2 * j + 1] = __fmul_rn(h0, h0);
    b[2 * j] = __fmul_rn(l1, l1);
    b[2 * j + 1] = __fmul_rn(h1, h1);
  }
  *reinterpret_cast<f32x4*>(sq + c) = a;
  *reinterpret_cast<f32x4*>(sq + c + 4) = b;
}

// The sequential fp32 sum of sq[0 .. H-1] in index order (one lane; H % 4 == 0).
// Reads run a batch ahead of the dependent adds.
__device__ __forceinline__ float sequential_sum(const float* sq, int H) {
  float ss = 0.f;
  int c = 0;
  for (; c + 32 <= H; c += 32) {
    f32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const f32x4*>(sq + c + 4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) ss = __fadd_rn(ss, v[i][j]);
  }
  for (; c < H; c += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(sq + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) ss = __fadd_rn(ss, v[j]);
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

// Lane 0 turns the squares in sq[0 .. H-1] into the row's scale, left in sq[H].
__device__ __forceinline__ float row_scale(float* sq, int H, float eps, int lane) {
  __syncthreads();
  if (lane == 0) sq[H] = rms_scale(sequential_sum(sq, H), H, eps);
  __syncthreads();
  return sq[H];
}

// grid T, block 64, dynamic LDS (H + 4) * 4 bytes.  Each lane keeps its chunks
// (channel chunk c = (lane + 64 i) * 8) in registers.  out may alias in.
__global__ __launch_bounds__(64) void rms_norm_kernel(int H, float eps, const uint16_t* in,
                                                      const float* __restrict__ gamma, uint16_t* out) {
  extern __shared__ __attribute__((aligned(16))) float sq[];
  const int t = blockIdx.x, lane = threadIdx.x;
  u32x4 v[kNormMaxChunks];
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = (lane + 64 * i) * 8;
    if (c < H) {
      v[i] = *reinterpret_cast<const u32x4*>(in + (size_t)t * H + c);
      store_squares8(sq, c, v[i]);
    }
  }
  const float r = row_scale(sq, H, eps, lane);
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = (lane + 64 * i) * 8;
    if (c < H) {
      float g[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) g[j] = gamma[c + j];
      *reinterpret_cast<u32x4*>(out + (size_t)t * H + c) = scale_gain8(v[i], r, g);
    }
  }
}

// Combine (as combine_kernel: fixed slot order, separately rounded mul/add) of
// token t, kept in registers (and written to moe_out if given), then post-norm
// and the residual mix into stream_out.  grid T, block 64, dynamic LDS
// (H + 4) * 4 bytes.  stream_out may alias stream_in: each lane reads its chunk
// of the stream before writing that chunk.
__global__ __launch_bounds__(64) void combine_norm_mix_kernel(int H, int K, const uint16_t* __restrict__ y,
                                                              const float* __restrict__ w,
                                                              const int32_t* __restrict__ pair_to_row,
                                                              float eps, const float* __restrict__ gamma, float a,
                                                              float b, const uint16_t* stream_in,
                                                              uint16_t* stream_out, uint16_t* __restrict__ moe_out) {
  extern __shared__ __attribute__((aligned(16))) float sq[];
  const int t = blockIdx.x, lane = threadIdx.x;
  u32x4 o[kNormMaxChunks];
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = (lane + 64 * i) * 8;
    if (c >= H) continue;
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
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[i][j] = static_cast<uint32_t>(f32_to_bf16(acc[2 * j])) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * j + 1])) << 16);
    if (moe_out) *reinterpret_cast<u32x4*>(moe_out + (size_t)t * H + c) = o[i];
    store_squares8(sq, c, o[i]);
  }
  const float r = row_scale(sq, H, eps, lane);
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = (lane + 64 * i) * 8;
    if (c >= H) continue;
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = gamma[c + j];
    const u32x4 p = scale_gain8(o[i], r, g);
    const u32x4 s = *reinterpret_cast<const u32x4*>(stream_in + (size_t)t * H + c);
    u32x4 n;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __fadd_rn(__fmul_rn(a, __uint_as_float(s[j] << 16)), __fmul_rn(b, __uint_as_float(p[j] << 16)));
      const float hi = __fadd_rn(__fmul_rn(a, __uint_as_float(s[j] & 0xFFFF0000u)),
                                 __fmul_rn(b, __uint_as_float(p[j] & 0xFFFF0000u)));
      n[j] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
    }
    *reinterpret_cast<u32x4*>(stream_out + (size_t)t * H + c) = n;
  }
}

hipError_t launch_rms_norm(int T, int H, float eps, const uint16_t* in, const float* gamma, uint16_t* out,
                           hipStream_t stream) {
  hipLaunchKernelGGL(rms_norm_kernel, dim3(T), dim3(64), (size_t)(H + 4) * 4, stream, H, eps, in, gamma, out);
  return hipGetLastError();
}

hipError_t launch_combine_norm_mix(const Shape& s, int T, const uint16_t* y, const float* w, const int32_t* pair_to_row,
                                   float eps, const float* gamma, float a, float b, const uint16_t* stream_in,
                                   uint16_t* stream_out, uint16_t* moe_out, hipStream_t stream) {
  hipLaunchKernelGGL(combine_norm_mix_kernel, dim3(T), dim3(64), (size_t)(s.H + 4) * 4, stream, s.H, s.K, y, w, pair_to_row,
                     eps, gamma, a, b, stream_in, stream_out, moe_out);
  return hipGetLastError();
}

}  // namespace beam
