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
//   router_logits: z partial sums over a K-split of the hidden dim on bf16
//                  MFMA: W_router (fp32) is split exactly into three bf16
//                  planes, w = hi + mid + lo, so every product x*w-part is
//                  exact (x is bf16) and the sums accumulate in fp32;
//   router_select: sum the partials in a fixed order, add the bias, sigmoid,
//                  then the selection in one wave (a workgroup per token at
//                  small T, a wave per token at large T).
#include "common.h"

namespace beam {

constexpr int kRTok = 128;   // tokens per workgroup: 4 waves x 2 row blocks of 16
constexpr int kRExp = 64;    // experts per workgroup: 4 column blocks of 16
constexpr int kRK = 32;      // k per step (one 16x16x32 MFMA)
constexpr int kRRow = 40;    // LDS row of one expert's 32 k: 32 bf16 + 8 pad (80 bytes: conflict-free reads)

// w = hi + mid + lo exactly, each a bf16: hi keeps w's top 8 significand bits
// (truncation), mid the top 8 of the remainder, lo the rest (at most 8
// significant bits).  Both subtractions are exact.  (Holds for |w| >= 2^-100;
// below that lo may lose bits to the fp32 subnormal range.)
__device__ __forceinline__ void split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t h = __float_as_uint(w) & 0xFFFF0000u;
  const float r1 = __fsub_rn(w, __uint_as_float(h));
  const uint32_t m = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = __fsub_rn(r1, __uint_as_float(m));
  hi = h >> 16;
  mid = m >> 16;
  lo = __float_as_uint(r2) >> 16;
}

// grid (ceil(T/128), ceil(E/64), ks); part ks covers k in [ks*kc, (ks+1)*kc), kc a multiple of 32.
// Wave w owns tokens [t0 + 32w, +32) and all 64 experts of the tile: per 32-k
// step two x fragments (straight from global memory: a lane reads 8
// consecutive k of one token row) and 3 planes x 4 expert blocks of W_router
// fragments from LDS, 24 MFMAs.  Each thread stages one expert x 8 k of the
// next step (8 loads, coalesced across the wave's 64 experts), splits them and
// writes the three planes; the LDS stage is double-buffered.
__global__ __launch_bounds__(256) void router_logits_kernel(int T, int H, int E, int kc,
                                                            const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][3][kRExp][kRRow];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int l16 = lane % 16, q = lane / 16;
  const int t0 = blockIdx.x * kRTok, e0 = blockIdx.y * kRExp, ks = blockIdx.z;
  const int kbeg = ks * kc, nst = kc / kRK;

  const uint16_t* xr[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int t = min(t0 + wave * 32 + m * 16 + l16, T - 1);   // rows past T read a valid row, never stored
    xr[m] = x + (size_t)t * H + kbeg + q * 8;
  }
  const int be = tid % kRExp, bk = (tid / kRExp) * 8;          // staged expert and first k of this thread
  const bool eok = e0 + be < E;
  const float* wcol = wr + (size_t)(kbeg + bk) * E + min(e0 + be, E - 1);
  float wv[8];
  auto load_b = [&](int st) {
#pragma unroll
    for (int j = 0; j < 8; ++j) wv[j] = eok ? wcol[((size_t)st * kRK + j) * E] : 0.f;
  };
  auto store_b = [&](int buf) {
    u32x4 pl[3];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t h0, m0, l0, h1, m1, l1;
      split3(wv[2 * j], h0, m0, l0);
      split3(wv[2 * j + 1], h1, m1, l1);
      pl[0][j] = h0 | (h1 << 16);
      pl[1][j] = m0 | (m1 << 16);
      pl[2][j] = l0 | (l1 << 16);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) *reinterpret_cast<u32x4*>(&ws[buf][p][be][bk]) = pl[p];
  };

  f32x4 acc[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_b(0);
  store_b(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) load_b(st + 1);
    bf16x8 a[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) a[m] = *reinterpret_cast<const bf16x8*>(xr[m] + st * kRK);
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(&ws[buf][p][n * 16 + l16][q * 8]);
#pragma unroll
        for (int m = 0; m < 2; ++m) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b, acc[m][n], 0, 0, 0);
      }
    if (st + 1 < nst) store_b(buf ^ 1);   // buffer buf^1 was last read in step st-1, before the barrier
    __syncthreads();
  }
  // C[r][c] of a 16x16 block sits in lane (c = l%16, r = 4q + i)
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + wave * 32 + m * 16 + q * 4 + i;
      if (t >= T) continue;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int e = e0 + n * 16 + l16;
        if (e < E) partial[((size_t)ks * T + t) * E + e] = acc[m][n][i];
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

// Small T (deep K-splits): one workgroup per token: thread e sums expert e's K-split partials in a
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
    int q = 0;
    for (; q + 8 <= ks; q += 8) {   // loads issued ahead of the adds, which stay in part order
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = p[(q + j) * stride];
#pragma unroll
      for (int j = 0; j < 8; ++j) z += v[j];
    }
    for (; q < ks; ++q) z += p[q * stride];
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

// Large T: one wave per token, four tokens per workgroup.  Lane l sums the K-split
// partials of experts l, l + 64, ... in a fixed order (coalesced across the
// lanes), adds the bias and takes the sigmoid; the wave then runs the
// group-limited selection on its token's scores in LDS.  The phases pass data
// through the wave's own LDS rows, ordered by wave-level fences.
constexpr int kSelTok = 4;          // tokens (waves) per workgroup
constexpr int kSelWaveMinT = 4096;  // from this many tokens the wave-per-token form runs

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
}

__global__ __launch_bounds__(kSelTok * kWave) void router_select_wave_kernel(
    int T, int E, int G, int Gk, int K, int ks, float alpha, const float* __restrict__ partial,
    const float* __restrict__ bias, int32_t* __restrict__ ids, float* __restrict__ wout) {
  __shared__ float s_sc_all[kSelTok][kMaxExperts];
  __shared__ float s_gs_all[kSelTok][64];
  __shared__ int s_keep_all[kSelTok][64];
  __shared__ float s_sel_all[kSelTok][kMaxTopK];
  const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int t = blockIdx.x * kSelTok + wv;
  if (t >= T) return;   // a whole wave; no workgroup barrier follows
  float* s_sc = s_sc_all[wv];
  float* s_gs = s_gs_all[wv];
  int* s_keep = s_keep_all[wv];
  float* s_sel = s_sel_all[wv];
  const size_t stride = (size_t)T * E;
  constexpr int kEL = kMaxExperts / kWave;   // experts per lane: lane, lane + 64, ...
  const float* p = partial + (size_t)t * E + lane;
  float z[kEL];
#pragma unroll
  for (int j = 0; j < kEL; ++j) z[j] = 0.f;
  int q = 0;
  for (; q + 8 <= ks; q += 8) {   // every expert's loads issued ahead of the adds, which stay in part order
    float v[kEL][8];
#pragma unroll
    for (int j = 0; j < kEL; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] = lane + kWave * j < E ? p[(q + i) * stride + kWave * j] : 0.f;
#pragma unroll
    for (int j = 0; j < kEL; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) z[j] += v[j][i];
  }
  for (; q < ks; ++q) {
    float v[kEL];
#pragma unroll
    for (int j = 0; j < kEL; ++j) v[j] = lane + kWave * j < E ? p[q * stride + kWave * j] : 0.f;
#pragma unroll
    for (int j = 0; j < kEL; ++j) z[j] += v[j];
  }
#pragma unroll
  for (int j = 0; j < kEL; ++j) {
    const int e = lane + kWave * j;
    if (e < E) {
      float zz = z[j];
      if (bias) zz += bias[e];
      s_sc[e] = 1.0f / (1.0f + expf(-zz));
    }
  }
  wave_lds_sync();
  const int gsz = E / G;
  // group score = top1 + top2 of the group's scores
  if (lane < G) {
    float a1 = -1.f, a2 = -1.f;
    for (int i = 0; i < gsz; ++i) {
      const float v = s_sc[lane * gsz + i];
      if (v > a1) { a2 = a1; a1 = v; } else if (v > a2) { a2 = v; }
    }
    s_gs[lane] = a1 + a2;
  }
  wave_lds_sync();
  // keep the Gk best groups (ties: lower group index)
  if (lane < G) {
    const float mine = s_gs[lane];
    int rank = 0;
    for (int g = 0; g < G; ++g) {
      const float o = s_gs[g];
      rank += (o > mine) || (o == mine && g < lane);
    }
    s_keep[lane] = rank < Gk;
  }
  wave_lds_sync();
  {
    // lane owns experts 4*lane .. 4*lane+3
    float sc[4];
    bool cand[4], sel[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      const bool ok = e < E;
      sc[j] = ok ? s_sc[e] : -1.f;
      cand[j] = ok && s_keep[e / gsz];
      sel[j] = false;
    }
    // K rounds of a wave-wide argmax over the remaining candidates (ties: lower id)
    for (int r = 0; r < K; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (cand[j] && !sel[j]) {
          const uint64_t key = (static_cast<uint64_t>(__float_as_uint(sc[j])) << 32) |
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
        s_sel[pos] = sc[j];
        ids[(size_t)t * K + pos] = lane * 4 + j;
        ++pos;
      }
    }
  }
  wave_lds_sync();
  if (lane < K) {
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
  // Both forms add the same partials in the same order.  At small T the K-split is deep (40 parts at 64
  // tokens) and a thread per expert keeps each chain short (decode: 12.7 against 19 us); at large T one
  // wave per token needs a quarter of the waves (8192 tokens: 31 against 48 us).
  if (T >= kSelWaveMinT) {
    hipLaunchKernelGGL(router_select_wave_kernel, dim3((T + kSelTok - 1) / kSelTok), dim3(kSelTok * kWave), 0,
                       stream, T, s.E, s.G, s.Gk, s.K, ks, s.alpha, partial, b, ids, w);
  } else {
    hipLaunchKernelGGL(router_select_kernel, dim3(T), dim3(256), 0, stream, T, s.E, s.G, s.Gk, s.K, ks, s.alpha,
                       partial, b, ids, w);
  }
  return hipGetLastError();
}

}  // namespace beam
