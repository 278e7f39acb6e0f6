// Grouped SwiGLU expert GEMMs on bf16 MFMA (v_mfma_f32_16x16x32_bf16), weight-streaming schedule.
//
// Each expert is a SwiGLU MLP (Reflection Beam 1.0 overview, section "Mixture of
// Experts"), with the SwiGLU product in FP32 (section "Residual stream"):
//   h = bf16( SiLU(x Wg^T) * (x Wu^T) )      gate/up kernel, fp32 epilogue
//   y = bf16( h Wd^T )                        down kernel
// Rows are the (token, slot) pairs routed to the expert, in permuted order;
// gate/up gathers x rows through sorted_pairs, down reads h rows in place.
//
// Work unit: one row tile of an expert (from the device-built tile list) times
// a block of output columns.  Each wave streams its weight rows straight from
// HBM into MFMA B-fragments (16 columns x 8 consecutive k per lane, 16-byte
// loads), so no LDS round trip sits between HBM and the matrix cores.  The
// reduction order inside an MFMA fragment is free, so A (x or h) and B use the
// same lane -> k mapping: lane l holds k in [k0 + 8*(l/16), +8), row/column l%16.
//
// FP8 weights (OCP e4m3) are converted exactly to bf16 in registers; the
// per-output-channel scale multiplies the fp32 accumulator in the epilogue.
#include "common.h"

namespace beam {

template <bool FP8>
struct WFrag;   // raw weight fragment of one lane for one k-step: 8 consecutive k of one output row
template <>
struct WFrag<false> {
  using T = bf16x8;
  static __device__ __forceinline__ T load(const void* base, size_t idx) {
    return *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(base) + idx);
  }
  static __device__ __forceinline__ bf16x8 cvt(T v) { return v; }
};
template <>
struct WFrag<true> {
  using T = u32x2;
  static __device__ __forceinline__ T load(const void* base, size_t idx) {
    return *reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(base) + idx);
  }
  static __device__ __forceinline__ bf16x8 cvt(T v) { return e4m3x8_to_bf16x8(v); }
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The streaming k-loop shared by both kernels.  Each k-step of 32 loads NB
// weight fragments (one per 16-column block, element offsets wofs[nb] + k) and
// MT activation fragments (arow[mt] + k), and issues MT*NB MFMAs.  Loads run D
// steps ahead of the MFMAs in a rolling register window, so every wave keeps
// D*NB weight loads in flight; the window is fully unrolled so each slot is a
// fixed register set.  Past the end, loads repeat the last step (harmless).
template <bool FP8, int MT, int NB, int D>
__device__ __forceinline__ void stream_k(int nsteps, const void* const (&wbase)[NB], const size_t (&wofs)[NB],
                                         const uint16_t* const (&arow)[MT], f32x4 (&acc)[MT][NB]) {
  using W = WFrag<FP8>;
  typename W::T wb[D][NB];
  bf16x8 ab[D][MT];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int st = min(j, nsteps - 1) * 32;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) wb[j][nb] = W::load(wbase[nb], wofs[nb] + st);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) ab[j][mt] = *reinterpret_cast<const bf16x8*>(arow[mt] + st);
  }
  const int nfull = nsteps / D;
  for (int w = 0; w < nfull; ++w) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 b = W::cvt(wb[j][nb]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][nb] = mfma16(ab[j][mt], b, acc[mt][nb]);
      }
      const int st = min((w + 1) * D + j, nsteps - 1) * 32;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wb[j][nb] = W::load(wbase[nb], wofs[nb] + st);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) ab[j][mt] = *reinterpret_cast<const bf16x8*>(arow[mt] + st);
    }
  }
  const int rem = nsteps - nfull * D;   // the last partial window is already loaded
#pragma unroll
  for (int j = 0; j < D - 1; ++j) {
    if (j < rem) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 b = W::cvt(wb[j][nb]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][nb] = mfma16(ab[j][mt], b, acc[mt][nb]);
      }
    }
  }
}

// Prefetch depth (k-steps in flight per wave) by row-tile count.
template <int MT>
struct Depth { static constexpr int value = MT == 1 ? 8 : (MT == 2 ? 6 : 4); };

// gate/up: grid (max_tiles, I/64), 4 waves; wave w owns columns [64*by + 16*w, +16) of gate and up.
// Rows past the tile's end read a valid row (the tile's first) and their
// outputs are discarded: an MFMA output row depends only on its own A row.
template <bool FP8, int MT>
__global__ __launch_bounds__(256) void gateup_stream_kernel(int H, int I, int K, const uint16_t* __restrict__ x,
                                                            const void* __restrict__ wg, const void* __restrict__ wu,
                                                            const float* __restrict__ sg, const float* __restrict__ su,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ sorted_pairs,
                                                            const int32_t* __restrict__ tiles,
                                                            const int32_t* __restrict__ ntiles,
                                                            uint16_t* __restrict__ h) {
  const int tile = blockIdx.x;
  if (tile >= ntiles[0]) return;
  const int e = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int lo = offsets[e];
  const int rows = min(offsets[e + 1] - lo - r0, 16 * MT);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int l16 = lane % 16, q = lane / 16;
  const int col = blockIdx.y * 64 + wave * 16 + l16;

  const uint16_t* xr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = mt * 16 + l16;
    const int tok = sorted_pairs[lo + r0 + (r < rows ? r : 0)] / K;
    xr[mt] = x + (size_t)tok * H + q * 8;
  }
  // gate and up rows of this lane's column
  const size_t wrow = ((size_t)e * I + col) * H + q * 8;
  const void* const wb[2] = {wg, wu};
  const size_t wofs[2] = {wrow, wrow};
  f32x4 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  stream_k<FP8, MT, 2, Depth<MT>::value>(H / 32, wb, wofs, xr, acc);

  float scg = 1.f, scu = 1.f;
  if constexpr (FP8) {
    scg = sg[(size_t)e * I + col];
    scu = su[(size_t)e * I + col];
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = mt * 16 + q * 4 + i;   // MFMA output row of this lane's i-th value
      if (r < rows) {
        const float g = acc[mt][0][i] * scg, u = acc[mt][1][i] * scu;
        h[(size_t)(lo + r0 + r) * I + col] = f32_to_bf16(silu(g) * u);
      }
    }
  }
}

// down: grid (max_tiles, H/128), 4 waves; wave w owns columns [128*by + 32*w, +32) as two 16-col blocks.
template <bool FP8, int MT>
__global__ __launch_bounds__(256) void down_stream_kernel(int H, int I, const uint16_t* __restrict__ hbuf,
                                                          const void* __restrict__ wd, const float* __restrict__ sd,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ tiles,
                                                          const int32_t* __restrict__ ntiles,
                                                          uint16_t* __restrict__ y) {
  const int tile = blockIdx.x;
  if (tile >= ntiles[0]) return;
  const int e = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int lo = offsets[e];
  const int rows = min(offsets[e + 1] - lo - r0, 16 * MT);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int l16 = lane % 16, q = lane / 16;
  const int c0 = blockIdx.y * 128 + wave * 32;
  if (c0 >= H) return;   // wave-uniform; H % 32 == 0 so both 16-column blocks are in range

  const uint16_t* hr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = mt * 16 + l16;
    hr[mt] = hbuf + (size_t)(lo + r0 + (r < rows ? r : 0)) * I + q * 8;
  }
  const size_t w0 = ((size_t)e * H + c0 + l16) * I + q * 8;
  const size_t wofs[2] = {w0, w0 + (size_t)16 * I};
  const void* const wb[2] = {wd, wd};
  f32x4 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  stream_k<FP8, MT, 2, Depth<MT>::value>(I / 32, wb, wofs, hr, acc);

  float s0 = 1.f, s1 = 1.f;
  if constexpr (FP8) {
    s0 = sd[(size_t)e * H + c0 + l16];
    s1 = sd[(size_t)e * H + c0 + 16 + l16];
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = mt * 16 + q * 4 + i;
      if (r < rows) {
        uint16_t* yr = y + (size_t)(lo + r0 + r) * H + c0 + l16;
        yr[0] = f32_to_bf16(acc[mt][0][i] * s0);
        yr[16] = f32_to_bf16(acc[mt][1][i] * s1);
      }
    }
  }
}

int expert_tile_rows(const Shape& s, int T) {
  const long mean = ((long)T * s.K + s.E - 1) / s.E;
  if (mean <= 12) return 16;
  if (mean <= 28) return 32;
  return 64;
}

template <bool FP8, int MT>
static hipError_t gateup_mt(const Shape& s, const uint16_t* x, const void* wg, const void* wu, const float* sg,
                            const float* su, const int32_t* offsets, const int32_t* sorted_pairs,
                            const int32_t* tiles, const int32_t* ntiles, int max_tiles, uint16_t* h,
                            hipStream_t stream) {
  hipLaunchKernelGGL((gateup_stream_kernel<FP8, MT>), dim3(max_tiles, s.I / 64), dim3(256), 0, stream, s.H, s.I,
                     s.K, x, wg, wu, sg, su, offsets, sorted_pairs, tiles, ntiles, h);
  return hipGetLastError();
}

template <bool FP8, int MT>
static hipError_t down_mt(const Shape& s, const uint16_t* h, const void* wd, const float* sd, const int32_t* offsets,
                          const int32_t* tiles, const int32_t* ntiles, int max_tiles, uint16_t* y,
                          hipStream_t stream) {
  hipLaunchKernelGGL((down_stream_kernel<FP8, MT>), dim3(max_tiles, (s.H + 127) / 128), dim3(256), 0, stream,
                     s.H, s.I, h, wd, sd, offsets, tiles, ntiles, y);
  return hipGetLastError();
}

hipError_t launch_gateup(const Shape& s, int T, const uint16_t* x, const void* wg, const void* wu,
                         const float* sg, const float* su, const int32_t* offsets, const int32_t* sorted_pairs,
                         const int32_t* tiles, const int32_t* ntiles, int max_tiles, uint16_t* h,
                         hipStream_t stream) {
  const int bm = expert_tile_rows(s, T);
#define BEAM_GU(F, M) gateup_mt<F, M>(s, x, wg, wu, sg, su, offsets, sorted_pairs, tiles, ntiles, max_tiles, h, stream)
  if (s.fp8) return bm == 16 ? BEAM_GU(true, 1) : bm == 32 ? BEAM_GU(true, 2) : BEAM_GU(true, 4);
  return bm == 16 ? BEAM_GU(false, 1) : bm == 32 ? BEAM_GU(false, 2) : BEAM_GU(false, 4);
#undef BEAM_GU
}

hipError_t launch_down(const Shape& s, int T, const uint16_t* h, const void* wd, const float* sd,
                       const int32_t* offsets, const int32_t* tiles, const int32_t* ntiles, int max_tiles,
                       uint16_t* y, hipStream_t stream) {
  const int bm = expert_tile_rows(s, T);
#define BEAM_DN(F, M) down_mt<F, M>(s, h, wd, sd, offsets, tiles, ntiles, max_tiles, y, stream)
  if (s.fp8) return bm == 16 ? BEAM_DN(true, 1) : bm == 32 ? BEAM_DN(true, 2) : BEAM_DN(true, 4);
  return bm == 16 ? BEAM_DN(false, 1) : bm == 32 ? BEAM_DN(false, 2) : BEAM_DN(false, 4);
#undef BEAM_DN
}

}  // namespace beam
