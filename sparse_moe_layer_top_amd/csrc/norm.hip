// RMSNorm before the MoE block, and the post-norm + constant-scale residual mix
// fused into the combine.
//
// Reflection Beam 1.0 overview, section "Residual stream": every sublayer is
// normalised before and after, the norms in FP32; the embedding is step 1 and
// at step k the sublayer output joins the stream with weight 1/sqrt(k) while
// the stream keeps sqrt((k-1)/k).  The norm is RMSNorm with a per-channel gain:
//   n = v / sqrt(mean(v^2) + eps),  out = bf16(n * gamma),
// every step one correctly rounded FP32 operation.  The sum of squares runs in a
// fixed order: the channels form 64 contiguous blocks of whole 8-channel chunks
// (block l: chunks [l*n/64, (l+1)*n/64), n = H/8), each summed in channel
// order, then the 64 block sums in block order.  The mix is
//   new = bf16( fp32(a * stream) + fp32(b * post) ),  a = sqrt((k-1)/k), b = 1/sqrt(k),
// with a and b rounded once to FP32 on the host.  Both kernels use one wave per
// token: every thread squares its channels (exact in FP32) into LDS, lane l of
// the first wave sums block l, lane 0 adds the block sums, and every thread
// applies the scale to the channels it holds in registers.
#include "beam_moe.h"
#include "common.h"
#include "rn_math.h"

namespace beam {

constexpr int kNormThreads = 256;                                          // one workgroup per token
constexpr int kNormMaxChunks = BEAM_MOE_MAX_NORM_HIDDEN / (kNormThreads * 8);   // 8-channel chunks per thread

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

// The squares in sq[0 .. H-1] -> the row's scale (left in sq[H]): lane l of
// wave 0 sums block l in channel order into sq[H + 4 + l], lane 0 adds the 64
// block sums in block order.  H % 8 == 0, so every block is whole 8-channel
// chunks.  Called by all threads of the workgroup.
__device__ __forceinline__ float row_scale(float* sq, int H, float eps) {
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int n = H / 8;
    const int lo = 8 * (tid * n / 64), hi = 8 * ((tid + 1) * n / 64);
    float part = 0.f;
    for (int c = lo; c < hi; c += 8) {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(sq + c);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(sq + c + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) part = __fadd_rn(part, v0[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) part = __fadd_rn(part, v1[j]);
    }
    sq[H + 4 + tid] = part;
  }
  __syncthreads();
  if (tid == 0) {
    float ss = 0.f;
    for (int l = 0; l < 64; ++l) ss = __fadd_rn(ss, sq[H + 4 + l]);
    sq[H] = rms_scale(ss, H, eps);
  }
  __syncthreads();
  return sq[H];
}

// grid T, block 256, dynamic LDS (H + 68) * 4 bytes.  Thread i keeps chunks
// c = (i + 256 j) * 8 in registers.  out may alias in.
__global__ __launch_bounds__(kNormThreads) void rms_norm_kernel(int H, float eps, const uint16_t* in,
                                                                const float* __restrict__ gamma, uint16_t* out) {
  extern __shared__ __attribute__((aligned(16))) float sq[];
  const int t = blockIdx.x, tid = threadIdx.x;
  u32x4 v[kNormMaxChunks];
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = (tid + kNormThreads * i) * 8;
    if (c < H) v[i] = *reinterpret_cast<const u32x4*>(in + (size_t)t * H + c);
  }
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = (tid + kNormThreads * i) * 8;
    if (c < H) store_squares8(sq, c, v[i]);
  }
  const float r = row_scale(sq, H, eps);
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = (tid + kNormThreads * i) * 8;
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
// and the residual mix into stream_out.  grid T, block 256, dynamic LDS
// (H + 68) * 4 bytes.  stream_out may alias stream_in: each thread reads its
// chunks of the stream before writing them.  The K slots' rows and weights are
// wave-uniform; each thread issues its chunks' loads of a slot together.
__global__ __launch_bounds__(kNormThreads) void combine_norm_mix_kernel(
    int H, int K, const uint16_t* __restrict__ y, const float* __restrict__ w, const int32_t* __restrict__ pair_to_row,
    float eps, const float* __restrict__ gamma, float a, float b, const uint16_t* stream_in, uint16_t* stream_out,
    uint16_t* __restrict__ moe_out) {
  extern __shared__ __attribute__((aligned(16))) float sq[];
  const int t = blockIdx.x, tid = threadIdx.x;
  float acc[kNormMaxChunks][8];
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  for (int k = 0; k < K; ++k) {
    const int p = t * K + k;
    const float wk = w[p];
    const uint16_t* yr = y + (size_t)pair_to_row[p] * H;
    u32x4 v[kNormMaxChunks];
#pragma unroll
    for (int i = 0; i < kNormMaxChunks; ++i) {
      const int c = (tid + kNormThreads * i) * 8;
      if (c < H) v[i] = *reinterpret_cast<const u32x4*>(yr + c);
    }
#pragma unroll
    for (int i = 0; i < kNormMaxChunks; ++i) {
      const int c = (tid + kNormThreads * i) * 8;
      if (c >= H) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][2 * j] = __fadd_rn(acc[i][2 * j], __fmul_rn(wk, __uint_as_float(v[i][j] << 16)));
        acc[i][2 * j + 1] = __fadd_rn(acc[i][2 * j + 1], __fmul_rn(wk, __uint_as_float(v[i][j] & 0xFFFF0000u)));
      }
    }
  }
  u32x4 o[kNormMaxChunks];
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = (tid + kNormThreads * i) * 8;
    if (c >= H) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[i][j] = static_cast<uint32_t>(f32_to_bf16(acc[i][2 * j])) | (static_cast<uint32_t>(f32_to_bf16(acc[i][2 * j + 1])) << 16);
    if (moe_out) *reinterpret_cast<u32x4*>(moe_out + (size_t)t * H + c) = o[i];
    store_squares8(sq, c, o[i]);
  }
  const float r = row_scale(sq, H, eps);
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = (tid + kNormThreads * i) * 8;
    if (c >= H) continue;
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = gamma[c + j];
    const u32x4 pv = scale_gain8(o[i], r, g);
    const u32x4 sv = *reinterpret_cast<const u32x4*>(stream_in + (size_t)t * H + c);
    u32x4 n;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __fadd_rn(__fmul_rn(a, __uint_as_float(sv[j] << 16)), __fmul_rn(b, __uint_as_float(pv[j] << 16)));
      const float hi = __fadd_rn(__fmul_rn(a, __uint_as_float(sv[j] & 0xFFFF0000u)),
                                 __fmul_rn(b, __uint_as_float(pv[j] & 0xFFFF0000u)));
      n[j] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
    }
    *reinterpret_cast<u32x4*>(stream_out + (size_t)t * H + c) = n;
  }
}

hipError_t launch_rms_norm(int T, int H, float eps, const uint16_t* in, const float* gamma, uint16_t* out,
                           hipStream_t stream) {
  hipLaunchKernelGGL(rms_norm_kernel, dim3(T), dim3(kNormThreads), (size_t)(H + 68) * 4, stream, H, eps, in, gamma, out);
  return hipGetLastError();
}

hipError_t launch_combine_norm_mix(const Shape& s, int T, const uint16_t* y, const float* w, const int32_t* pair_to_row,
                                   float eps, const float* gamma, float a, float b, const uint16_t* stream_in,
                                   uint16_t* stream_out, uint16_t* moe_out, hipStream_t stream) {
  hipLaunchKernelGGL(combine_norm_mix_kernel, dim3(T), dim3(kNormThreads), (size_t)(s.H + 68) * 4, stream, s.H, s.K, y, w, pair_to_row,
                     eps, gamma, a, b, stream_in, stream_out, moe_out);
  return hipGetLastError();
}

}  // namespace beam
