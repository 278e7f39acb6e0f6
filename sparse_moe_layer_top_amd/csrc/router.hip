// Router: fp32 logits over all experts, sigmoid, group-limited top-k, normalised weights.
//
// Reflection Beam 1.0 overview (agentlenshq.com), section "Mixture of Experts":
// a sigmoid scores all experts; experts are split into groups, each group is
// ranked by the sum of its top-2 scores, the best groups are kept and the best
// K experts inside them chosen; weights are the chosen scores normalised and
// scaled by alpha.  The router is computed in FP32 (same page, section
// "Residual stream").
//
// Two kernels:
//   router_logits: z partial sums over a K-split of the hidden dim, fp32 FMA,
//                  LDS-staged 64-token x 64-expert tiles;
//   router_select: one workgroup per token: sum the partials in a fixed order,
//                  add the bias, sigmoid, then the selection in one wave.
#include "common.h"

namespace beam {

constexpr int kRTok = 64, kRExp = 64, kRK = 32;

__global__ __launch_bounds__(256) void router_logits_kernel(int T, int H, int E, int kc,
                                                            const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) float xs[kRK][kRTok + 4];
  __shared__ __attribute__((aligned(16))) float ws[kRK][kRExp + 4];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRTok, e0 = blockIdx.y * kRExp, ks = blockIdx.z;
  const int kbeg = ks * kc, kend = kbeg + kc;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  const int lt = tid / 4, lp = tid % 4;   // x tile: token, 8-wide k part
  const int wk = tid / 8, wp = tid % 8;   // w tile: k row, 8-wide expert part
  const bool xok = (t0 + lt) < T;
  const uint16_t* xrow = x + (size_t)(xok ? t0 + lt : 0) * H;
  const bool wvec = (E % 4) == 0 && (e0 + wp * 8 + 8) <= E;

  for (int k0 = kbeg; k0 < kend; k0 += kRK) {
    // stage x (bf16 -> fp32, transposed to [k][token]) and W_router ([k][expert])
    u32x4 xv = {0u, 0u, 0u, 0u};
    if (xok) xv = *reinterpret_cast<const u32x4*>(xrow + k0 + lp * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xs[lp * 8 + 2 * j][lt] = __uint_as_float(xv[j] << 16);
      xs[lp * 8 + 2 * j + 1][lt] = __uint_as_float(xv[j] & 0xFFFF0000u);
    }
    const float* wrow = wr + (size_t)(k0 + wk) * E + e0 + wp * 8;
    if (wvec) {
      f32x4 a = *reinterpret_cast<const f32x4*>(wrow);
      f32x4 b = *reinterpret_cast<const f32x4*>(wrow + 4);
      *reinterpret_cast<f32x4*>(&ws[wk][wp * 8]) = a;
      *reinterpret_cast<f32x4*>(&ws[wk][wp * 8 + 4]) = b;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) ws[wk][wp * 8 + j] = (e0 + wp * 8 + j < E) ? wrow[j] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < kRK; ++k) {
      f32x4 a = *reinterpret_cast<const f32x4*>(&xs[k][ty * 4]);
      f32x4 b = *reinterpret_cast<const f32x4*>(&ws[k][tx * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) partial[((size_t)ks * T + t) * E + e] = acc[i][j];
    }
  }
}

// 64-bit max across the wave (keys are unique, so the result is exact).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m);
    uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// One workgroup per token: thread e sums expert e's K-split partials in a
// fixed order (coalesced across threads), adds the bias and takes the sigmoid;
// wave 0 then runs the group-limited selection on the scores in LDS.
__global__ __launch_bounds__(256) void router_select_kernel(int T, int E, int G, int Gk, int K, int ks,
                                                            float alpha, const float* __restrict__ partial,
                                                            const float* __restrict__ bias,
                                                            int32_t* __restrict__ ids, float* __restrict__ wout) {
  __shared__ float s_sc[kMaxExperts];
  __shared__ float s_gs[64];
  __shared__ int s_keep[64];
  __shared__ float s_sel[kMaxTopK];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < E) {
    const float* p = partial + (size_t)t * E + tid;
    const size_t stride = (size_t)T * E;
    float z = 0.f;
    for (int q = 0; q < ks; ++q) z += p[q * stride];
    if (bias) z += bias[tid];
    s_sc[tid] = 1.0f / (1.0f + expf(-z));
  }
  __syncthreads();
  const int lane = tid % kWave;
  const bool w0 = tid < kWave;   // wave 0 selects; the others only join the barriers
  const int gsz = E / G;
  // group score = top1 + top2 of the group's scores
  if (w0 && lane < G) {
    float a1 = -1.f, a2 = -1.f;
    for (int i = 0; i < gsz; ++i) {
      const float v = s_sc[lane * gsz + i];
      if (v > a1) { a2 = a1; a1 = v; } else if (v > a2) { a2 = v; }
    }
    s_gs[lane] = a1 + a2;
  }
  __syncthreads();
  // keep the Gk best groups (ties: lower group index)
  if (w0 && lane < G) {
    const float mine = s_gs[lane];
    int rank = 0;
    for (int g = 0; g < G; ++g) {
      const float o = s_gs[g];
      rank += (o > mine) || (o == mine && g < lane);
    }
    s_keep[lane] = rank < Gk;
  }
  __syncthreads();
  if (w0) {
    // lane owns experts 4*lane .. 4*lane+3
    float s[4];
    bool cand[4], sel[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      const bool ok = e < E;
      s[j] = ok ? s_sc[e] : -1.f;
      cand[j] = ok && s_keep[e / gsz];
      sel[j] = false;
    }
    // K rounds of a wave-wide argmax over the remaining candidates (ties: lower id)
    for (int r = 0; r < K; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (cand[j] && !sel[j]) {
          const uint64_t key = (static_cast<uint64_t>(__float_as_uint(s[j])) << 32) |
                               (0xFFFFFFFFu - static_cast<uint32_t>(lane * 4 + j));
          best = key > best ? key : best;
        }
      }
      best = wave_max_u64(best);
      const uint32_t win = 0xFFFFFFFFu - static_cast<uint32_t>(best);
      if ((win >> 2) == static_cast<uint32_t>(lane)) sel[win & 3] = true;
    }
    // slot of each chosen expert = number of chosen experts with a lower id
    uint64_t m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = __ballot(sel[j]);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int pos = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) pos += __popcll(m[j] & below);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (sel[j]) {
        s_sel[pos] = s[j];
        ids[(size_t)t * K + pos] = lane * 4 + j;
        ++pos;
      }
    }
  }
  __syncthreads();
  if (w0 && lane < K) {
    float den = 0.f;
    for (int k = 0; k < K; ++k) den += s_sel[k];   // sequential, ascending expert id
    wout[(size_t)t * K + lane] = (s_sel[lane] / den) * alpha;
  }
}

hipError_t launch_router_logits(const Shape& s, int T, int ks, const uint16_t* x, const float* wr,
                                float* partial, hipStream_t stream) {
  dim3 grid((T + kRTok - 1) / kRTok, (s.E + kRExp - 1) / kRExp, ks);
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, stream, T, s.H, s.E, s.H / ks, x, wr, partial);
  return hipGetLastError();
}

hipError_t launch_router_select(const Shape& s, int T, int ks, const float* partial, const float* b,
                                int32_t* ids, float* w, hipStream_t stream) {
  dim3 grid(T);
  hipLaunchKernelGGL(router_select_kernel, grid, dim3(256), 0, stream, T, s.E, s.G, s.Gk, s.K, ks, s.alpha,
                     partial, b, ids, w);
  return hipGetLastError();
}

}  // namespace beam
