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
// loads), so no LDS round trip sits between HBM and the matrix cores; the
// activation rows (x or h), the same for the workgroup's four waves, reach the
// MFMAs through a small LDS window.  The reduction order inside an MFMA
// fragment is free, so A and B use the same lane -> k mapping: lane l holds k
// in [k0 + 8*(l/16), +8), row/column l%16.
//
// FP8 weights (OCP e4m3) are converted exactly to bf16 in registers; the
// per-output-channel scale multiplies the fp32 accumulator in the epilogue.
// MXFP4 weights (E2M1, two per byte, one E8M0 scale per 32 inputs) are
// converted with their block scale to bf16 in registers (exact: a power of
// two times a 2-bit-significand value); one 16-byte load holds 32 values, a
// whole scale block.
#include <type_traits>

#include "common.h"

namespace beam {

enum { kWBF16 = 0, kWFP8 = 1, kWMX = 2 };

template <int WT>
struct WFrag;   // one lane's 16-byte weight load per k-step and its conversion to MFMA B-fragments
template <>
struct WFrag<kWBF16> {
  using E = uint16_t;
  static constexpr int SK = 32;     // k per step: one 16x16x32 MFMA
  static constexpr int SE = 32;     // weight elements (of type E) per row per step
  static constexpr bool kBlockScale = false;
  static __device__ __forceinline__ bf16x8 frag(u32x4 v, int, float) { return __builtin_bit_cast(bf16x8, v); }
};
template <>
struct WFrag<kWFP8> {
  using E = uint8_t;
  static constexpr int SK = 64;     // 16 e4m3 bytes feed two MFMAs
  static constexpr int SE = 64;
  static constexpr bool kBlockScale = false;
  static __device__ __forceinline__ bf16x8 frag(u32x4 v, int a, float) {
    return e4m3x8_to_bf16x8(a == 0 ? u32x2{v[0], v[1]} : u32x2{v[2], v[3]});
  }
};
template <>
struct WFrag<kWMX> {
  using E = uint8_t;
  static constexpr int SK = 128;    // 16 bytes = 32 E2M1 values per lane feed four MFMAs
  static constexpr int SE = 64;     // bytes per row per step
  static constexpr bool kBlockScale = true;
  static __device__ __forceinline__ bf16x8 frag(u32x4 v, int a, float scale) { return e2m1x8_to_bf16x8(v[a], scale); }
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Scale bytes of a window: D consecutive k-steps x 4 lane quads, one byte each, contiguous in an
// MXFP4 scale row, fetched with one D-dword load.
template <int D>
struct ScaleVec;
template <>
struct ScaleVec<1> { using T = uint32_t; };
template <>
struct ScaleVec<2> { using T = u32x2; };
template <>
struct ScaleVec<4> { using T = u32x4; };

constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);   // s_waitcnt lgkmcnt(0), vmcnt not waited on

// Activation fragments of one window: D steps x MT row blocks x SK/32 MFMA k-slices, each 1 KB
// (64 lanes x 16 bytes, laid out so that lane l reads slot[l]: conflict-free).  The four waves of a
// workgroup share one copy; wave w loads fragments w, w+4, ... (past F it reloads a valid one
// into a spare slot, so every wave runs the same straight-line code).
template <int WT, int MT, int D>
struct AWin {
  static constexpr int NA = WFrag<WT>::SK / 32;
  static constexpr int F = D * MT * NA;
  static constexpr int FW = (F + 3) / 4;
  static constexpr int SLOTS = 4 * FW;
};

// The streaming k-loop shared by both kernels.  A step covers SK k-values.
// Lane (row/column l%16, quad q = l/16) owns k in [step*SK + q*SK/4, +SK/4):
// one 16-byte weight load per weight block (NB blocks of 16 output columns)
// per step, wst weight elements after the last (row order: the next 64 bytes
// of the row; fragment order: the block's next 1 KB slice); wrow/arow already
// include the lane's offset.  srow (MXFP4) is the row's scale base, t0 the
// first step's index: step t's four scale bytes sit at 4t in row order, and
// at 256(t/4) + 4(t%4) in fragment order (srow there already includes the
// row's 16 bytes within each 256-byte slice of its 16-row block).
//
// Weights go straight from HBM into registers in bursts: a window of D steps
// is issued back to back (each weight row sees D*64 contiguous bytes requested
// together, which HBM serves better than the same loads spread out), and
// windows are double-buffered: window w+1 is in flight while window w feeds
// the MFMAs.  Activations (L2 hits, the same for every wave of the workgroup)
// do not sit in registers for a whole window: each wave loads a quarter of
// the next window's fragments into a few staging registers together with the
// weight burst, writes them to LDS after computing the current window, and
// one barrier per window publishes them.  That keeps per-lane registers to
// the weight ring, which sets how many bytes each CU keeps in flight.
// sched_barrier fences keep the compiler from reordering the bursts.
template <int WT, int MT, int NB, int D>
__device__ __forceinline__ void stream_k(int nsteps, int wst, int t0, int sfrag, int wave, int lane,
                                         const typename WFrag<WT>::E* const (&wrow)[NB],
                                         const uint8_t* const (&srow)[NB], const uint16_t* const (&arow)[MT],
                                         u32x4 (*lds)[AWin<WT, MT, D>::SLOTS][kWave], f32x4 (&acc)[MT][NB]) {
  using W = WFrag<WT>;
  using A = AWin<WT, MT, D>;
  constexpr int SK = W::SK, NA = A::NA;
  const int q = lane / 16;
  const uint16_t* mine[A::FW];   // this lane's address of each fragment this wave loads (window 0)
#pragma unroll
  for (int i = 0; i < A::FW; ++i) {
    const int f = (wave + 4 * i) % A::F;
    const int fj = f / (MT * NA), fm = (f / NA) % MT, fa = f % NA;
    const uint16_t* p = arow[0];
#pragma unroll
    for (int m = 1; m < MT; ++m) p = fm == m ? arow[m] : p;
    mine[i] = p + fj * SK + fa * 8;
  }
  u32x4 wb[2][D][NB];
  uint32_t sb[2][W::kBlockScale ? NB : 1][D];
  u32x4 st[A::FW];
  const int nwin = nsteps / D;
  auto load = [&](int buf, int w) {
    const int base = w * D;
#pragma unroll
    for (int i = 0; i < A::FW; ++i) st[i] = *reinterpret_cast<const u32x4*>(mine[i] + base * SK);
#pragma unroll
    for (int j = 0; j < D; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wb[buf][j][nb] = *reinterpret_cast<const u32x4*>(wrow[nb] + (size_t)(base + j) * wst);
    if constexpr (W::kBlockScale) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int t = t0 + base;
        const int so = sfrag ? (t >> 2) * 256 + (t & 3) * 4 : t * 4;
        const auto v = *reinterpret_cast<const typename ScaleVec<D>::T*>(srow[nb] + so);
        if constexpr (D == 1) {
          sb[buf][nb][0] = v;
        } else {
#pragma unroll
          for (int j = 0; j < D; ++j) sb[buf][nb][j] = v[j];
        }
      }
    }
  };
  auto publish = [&](int buf) {   // staged fragments -> LDS, then every wave's are visible
#pragma unroll
    for (int i = 0; i < A::FW; ++i) lds[buf][wave + 4 * i][lane] = st[i];
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int j = 0; j < D; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float sc = 1.f;
        if constexpr (W::kBlockScale) sc = e8m0_to_f32((sb[buf][nb][j] >> (8 * q)) & 0xFFu);
#pragma unroll
        for (int a = 0; a < NA; ++a) {
          const bf16x8 b = W::frag(wb[buf][j][nb], a, sc);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const bf16x8 af = __builtin_bit_cast(bf16x8, lds[buf][(j * MT + mt) * NA + a][lane]);
            acc[mt][nb] = mfma16(af, b, acc[mt][nb]);
          }
        }
      }
  };
  load(0, 0);
  publish(0);
  __builtin_amdgcn_sched_barrier(0);
  int w = 0;
  for (; w + 2 < nwin; w += 2) {
    load(1, w + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    __builtin_amdgcn_sched_barrier(0);
    publish(1);
    __builtin_amdgcn_sched_barrier(0);
    load(0, w + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    __builtin_amdgcn_sched_barrier(0);
    publish(0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the last one or two windows, with nothing loaded past the end
  if (w + 1 < nwin) {
    load(1, w + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    __builtin_amdgcn_sched_barrier(0);
    publish(1);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
  } else {
    compute(0);
  }
}

// Columns per wave (G blocks of 16 per matrix) and the burst-depth caps, per
// weight type and row-tile count, from sweeps of the real shapes at T = 64,
// 512 and 2048: depth 4 wins at 16-row tiles for every weight type (bf16
// gate/up 6.1 TB/s), 2 at 64-row tiles; one column block per wave wherever
// measured.
template <int WT, int MT>
struct StreamShape {
  static constexpr int kGateUpG = 1;
  static constexpr int kDownG = 1;
  static constexpr int kGateUpDepth = MT == 4 ? 2 : (WT == kWFP8 && MT == 2 ? 2 : 4);
  static constexpr int kDownDepth = MT == 4 ? 2 : (MT == 2 && WT != kWBF16 ? 2 : 4);
};

// gate/up: grid (ceil(I / 64G), max_tiles, kparts), 4 waves; workgroup (bx, by)
// takes column block bx of row tile by, and wave w owns columns
// [64G*bx + 16G*w, +16G) of gate and of up.  Column blocks vary fastest, so the
// workgroups in flight together stream one expert's rows at many offsets rather
// than the same offset of every expert's matrix (expert matrices are a multiple
// of 1 MiB apart and the latter lands them on the same HBM channels: 5% slower
// with the router's own expert ids).  With kparts > 1 part z covers
// reduction steps [z*n, (z+1)*n) and writes raw fp32 sums; swiglu_reduce_kernel
// adds the parts in z order and applies the SwiGLU (the dense path at small T).  Rows past the tile's end read a
// valid row (the tile's first) and their outputs are discarded: an MFMA
// output row depends only on its own A row.  Waves past the last column
// stream valid rows (the workgroup shares a barrier) and store nothing.
template <int WT, int MT, int G, int D>
__global__ __launch_bounds__(256) void gateup_stream_kernel(int H, int I, int K, const uint16_t* __restrict__ x,
                                                            const void* __restrict__ wg, const void* __restrict__ wu,
                                                            const void* __restrict__ sg, const void* __restrict__ su,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ sorted_pairs,
                                                            const int32_t* __restrict__ tiles,
                                                            const int32_t* __restrict__ ntiles,
                                                            uint16_t* __restrict__ h, int kparts, int nrows,
                                                            float* __restrict__ part, int packed) {
  using W = WFrag<WT>;
  __shared__ u32x4 lds[2][AWin<WT, MT, D>::SLOTS][kWave];
  const int tile = blockIdx.y;
  if (tile >= ntiles[0]) return;   // uniform over the workgroup
  const int e = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int lo = offsets[e];
  const int rows = min(offsets[e + 1] - lo - r0, 16 * MT);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int l16 = lane % 16, q = lane / 16;
  const int colw = blockIdx.x * 64 * G + wave * 16 * G;
  const bool active = colw < I;
  const int col0 = active ? colw : 0;
  const int qa = q * (W::SK / 4), qw = q * (W::SE / 4);   // lane quad offsets: activations (k), weights (E units)
  const int nsteps = H / W::SK / kparts;
  const size_t zs = (size_t)blockIdx.z * nsteps;   // first step of this part (0 unless split)

  const uint16_t* xr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = mt * 16 + l16;
    const int tok = sorted_pairs[lo + r0 + (r < rows ? r : 0)] / K;
    xr[mt] = x + (size_t)tok * H + qa + zs * W::SK;
  }
  using WE = typename W::E;
  const size_t HE = (size_t)H * W::SE / W::SK;          // a weight row in E units
  const WE* wr[2 * G];
  const uint8_t* sr[2 * G];
#pragma unroll
  for (int g = 0; g < 2 * G; ++g) {
    const size_t row0 = (size_t)e * I + col0 + (g % G) * 16, row = row0 + l16;   // the block's first row, the lane's
    wr[g] = static_cast<const WE*>(g < G ? wg : wu) +
            (packed ? row0 * HE + lane * (16 / sizeof(WE)) + zs * W::SE * 16 : row * HE + qw + zs * W::SE);
    sr[g] = W::kBlockScale ? static_cast<const uint8_t*>(g < G ? sg : su) +
                                 (packed ? row0 * (H / 32) + l16 * 16 : row * (H / 32))
                           : nullptr;
  }
  f32x4 acc[MT][2 * G];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int g = 0; g < 2 * G; ++g) acc[mt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
  stream_k<WT, MT, 2 * G, D>(nsteps, packed ? 16 * W::SE : W::SE, (int)zs, packed, wave, lane, wr, sr, xr, lds, acc);
  if (!active) return;
  if (kparts > 1) {   // raw fp32 sums of this part: gate at part[z][row][col], up at part[z][row][I + col]
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mt * 16 + q * 4 + i;
          if (r >= rows) continue;
          float* pr = part + ((size_t)blockIdx.z * nrows + lo + r0 + r) * (2 * (size_t)I) + col0 + g * 16 + l16;
          pr[0] = acc[mt][g][i];
          pr[I] = acc[mt][G + g][i];
        }
    return;
  }

#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int col = col0 + g * 16 + l16;
    float scg = 1.f, scu = 1.f;
    if constexpr (WT == kWFP8) {
      scg = static_cast<const float*>(sg)[(size_t)e * I + col];
      scu = static_cast<const float*>(su)[(size_t)e * I + col];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + q * 4 + i;   // MFMA output row of this lane's i-th value
        if (r < rows) {
          const float gv = acc[mt][g][i] * scg, uv = acc[mt][G + g][i] * scu;
          h[(size_t)(lo + r0 + r) * I + col] = f32_to_bf16(silu(gv) * uv);
        }
      }
    }
  }
}

// down: grid (ceil(H / 128G), max_tiles, kparts), columns fastest as for
// gate/up; wave w owns columns [128G*bx + 32G*w, +32G).  With kparts > 1 (grid z), part z covers reduction
// steps [z*n, (z+1)*n) and writes its raw fp32 sums to part[z][row][col];
// splitk_reduce_kernel adds the parts in z order.  Used when one expert's rows
// are too few to fill the chip.
template <int WT, int MT, int G, int D>
__global__ __launch_bounds__(256) void down_stream_kernel(int H, int I, const uint16_t* __restrict__ hbuf,
                                                          const void* __restrict__ wd, const void* __restrict__ sd,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ tiles,
                                                          const int32_t* __restrict__ ntiles,
                                                          uint16_t* __restrict__ y, int kparts, int nrows,
                                                          float* __restrict__ part, int packed) {
  using W = WFrag<WT>;
  __shared__ u32x4 lds[2][AWin<WT, MT, D>::SLOTS][kWave];
  const int tile = blockIdx.y;
  if (tile >= ntiles[0]) return;   // uniform over the workgroup
  const int e = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int lo = offsets[e];
  const int rows = min(offsets[e + 1] - lo - r0, 16 * MT);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int l16 = lane % 16, q = lane / 16;
  const int cw = blockIdx.x * 128 * G + wave * 32 * G;
  const bool active = cw < H;
  const int c0 = active ? cw : 0;
  const int qa = q * (W::SK / 4), qw = q * (W::SE / 4);
  const int nsteps = I / W::SK / kparts;
  const size_t zs = (size_t)blockIdx.z * nsteps;   // first step of this part (0 unless split)

  const uint16_t* hr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = mt * 16 + l16;
    hr[mt] = hbuf + (size_t)(lo + r0 + (r < rows ? r : 0)) * I + qa + zs * W::SK;
  }
  using WE = typename W::E;
  const size_t IE = (size_t)I * W::SE / W::SK;          // a weight row in E units
  const WE* wr[2 * G];
  const uint8_t* sr[2 * G];
#pragma unroll
  for (int g = 0; g < 2 * G; ++g) {
    const size_t row0 = (size_t)e * H + c0 + g * 16, row = row0 + l16;
    wr[g] = static_cast<const WE*>(wd) +
            (packed ? row0 * IE + lane * (16 / sizeof(WE)) + zs * W::SE * 16 : row * IE + qw + zs * W::SE);
    sr[g] = W::kBlockScale ? static_cast<const uint8_t*>(sd) + (packed ? row0 * (I / 32) + l16 * 16 : row * (I / 32))
                           : nullptr;
  }
  f32x4 acc[MT][2 * G];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int g = 0; g < 2 * G; ++g) acc[mt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
  stream_k<WT, MT, 2 * G, D>(nsteps, packed ? 16 * W::SE : W::SE, (int)zs, packed, wave, lane, wr, sr, hr, lds, acc);
  if (!active) return;

#pragma unroll
  for (int g = 0; g < 2 * G; ++g) {
    const int col = c0 + g * 16 + l16;
    float sc = 1.f;
    if constexpr (WT == kWFP8) sc = static_cast<const float*>(sd)[(size_t)e * H + col];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + q * 4 + i;
        if (r >= rows) continue;
        if (kparts > 1)
          part[((size_t)blockIdx.z * nrows + lo + r0 + r) * H + col] = acc[mt][g][i];
        else
          y[(size_t)(lo + r0 + r) * H + col] = f32_to_bf16(acc[mt][g][i] * sc);
      }
    }
  }
}

int expert_tile_rows(const Shape& s, int T) {
  if (wide_schedule(s, T) != kWideNone) return wide_tile_rows(s, T);
  if (use_tiled(s, T)) return tiled_tile_rows();
  const long mean = ((long)T * s.K + s.E - 1) / s.E;
  if (mean <= 12) return 16;
  if (mean <= 28) return 32;
  return 64;
}

// Row tiles index the grid's y dimension (at most 65535).  The streaming path
// stays far below it: 16- and 32-row tiles only serve T*K/E <= 28, and 64-row
// tiles at the largest T give T*K/64 + E = 33024.
constexpr int kMaxGridY = 65535;

// Largest D in {4, 2, 1}, at most cap, dividing nsteps.  (An MXFP4 scale
// window of D dwords is then aligned: a scale row holds 4 * nsteps bytes.)
static int pick_depth(int nsteps, int cap) {
  for (int d = cap; d > 1; d /= 2)
    if (nsteps % d == 0) return d;
  return 1;
}

template <int WT, int MT, int G, int D>
static hipError_t gateup_launch(const Shape& s, const uint16_t* x, const void* wg, const void* wu, const void* sg,
                                const void* su, const int32_t* offsets, const int32_t* sorted_pairs,
                                const int32_t* tiles, const int32_t* ntiles, int max_tiles, uint16_t* h,
                                int kparts, int nrows, float* part, hipStream_t stream) {
  hipLaunchKernelGGL((gateup_stream_kernel<WT, MT, G, D>), dim3((s.I + 64 * G - 1) / (64 * G), max_tiles, kparts),
                     dim3(256), 0, stream, s.H, s.I, s.K, x, wg, wu, sg, su, offsets, sorted_pairs, tiles, ntiles, h,
                     kparts, nrows, part, s.packed);
  return hipGetLastError();
}

// h[row][c] = bf16( SiLU(G * sg[c]) * (U * su[c]) ), G and U the sums of the
// parts in z order (fp8: the per-row scales; NULL: none).  The dense path's
// single expert: the scale of intermediate column c is sg[c] / su[c].
__global__ __launch_bounds__(256) void swiglu_reduce_kernel(int nrows, int I, int kparts, const float* __restrict__ part,
                                                            const float* __restrict__ sg, const float* __restrict__ su,
                                                            uint16_t* __restrict__ h) {
  const size_t n = (size_t)nrows * I, stride = (size_t)nrows * 2 * I;
  for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += (size_t)gridDim.x * 256 * 4) {
    const size_t row = i / I, c = i % I;
    const float* pg = part + row * 2 * I + c;
    f32x4 g = *reinterpret_cast<const f32x4*>(pg), u = *reinterpret_cast<const f32x4*>(pg + I);
    for (int z = 1; z < kparts; ++z) {
      const f32x4 gz = *reinterpret_cast<const f32x4*>(pg + z * stride);
      const f32x4 uz = *reinterpret_cast<const f32x4*>(pg + z * stride + I);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        g[j] = __fadd_rn(g[j], gz[j]);
        u[j] = __fadd_rn(u[j], uz[j]);
      }
    }
    u32x2 o;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float hv[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int cc = (int)c + 2 * j + m;
        const float gv = g[2 * j + m] * (sg ? sg[cc] : 1.f), uv = u[2 * j + m] * (su ? su[cc] : 1.f);
        hv[m] = silu(gv) * uv;
      }
      o[j] = static_cast<uint32_t>(f32_to_bf16(hv[0])) | (static_cast<uint32_t>(f32_to_bf16(hv[1])) << 16);
    }
    *reinterpret_cast<u32x2*>(h + i) = o;
  }
}

template <int WT, int MT, int G, int D>
static hipError_t down_launch(const Shape& s, const uint16_t* h, const void* wd, const void* sd,
                              const int32_t* offsets, const int32_t* tiles, const int32_t* ntiles, int max_tiles,
                              uint16_t* y, int kparts, int nrows, float* part, hipStream_t stream) {
  hipLaunchKernelGGL((down_stream_kernel<WT, MT, G, D>), dim3((s.H + 128 * G - 1) / (128 * G), max_tiles, kparts),
                     dim3(256), 0, stream, s.H, s.I, h, wd, sd, offsets, tiles, ntiles, y, kparts, nrows, part,
                     s.packed);
  return hipGetLastError();
}

// y[row][col] = bf16( (part[0] + part[1] + ... + part[kparts-1]) * scale[col] ), parts added in order.
// One expert (the dense path): the fp8 scale of output column col is sd[col] (NULL: no scale).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(int nrows, int H, int kparts, const float* __restrict__ part,
                                                            const float* __restrict__ sd, uint16_t* __restrict__ y) {
  const size_t n = (size_t)nrows * H;
  for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += (size_t)gridDim.x * 256 * 4) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
    for (int z = 1; z < kparts; ++z) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(part + (size_t)z * n + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __fadd_rn(acc[j], v[j]);
    }
    u32x2 o;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = (int)((i + 2 * j) % H);
      const float a = sd ? __fmul_rn(acc[2 * j], sd[c]) : acc[2 * j];
      const float b = sd ? __fmul_rn(acc[2 * j + 1], sd[c + 1]) : acc[2 * j + 1];
      o[j] = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
    }
    *reinterpret_cast<u32x2*>(y + i) = o;
  }
}

static int weight_type_of(const Shape& s) { return s.mx ? kWMX : (s.fp8 ? kWFP8 : kWBF16); }

static int steps_per_k(const Shape& s, int K) {
  return K / (s.mx ? WFrag<kWMX>::SK : (s.fp8 ? WFrag<kWFP8>::SK : WFrag<kWBF16>::SK));
}

// Reduction parts for the dense path's down GEMM: the fewest parts giving about
// 1024 workgroups, each part a multiple of 4 steps where the step count allows
// (keeping the deepest burst schedule); 1 when the row tiles alone fill the GPU.
int down_kparts(const Shape& s, int T) {
  if (!s.dense || use_tiled(s, T)) return 1;
  const int bm = expert_tile_rows(s, T);
  const long wgs = (long)((T + bm - 1) / bm) * ((s.H + 127) / 128);
  const int steps = steps_per_k(s, s.I);
  const int grain = steps % 4 == 0 ? 4 : (steps % 2 == 0 ? 2 : 1);
  int best = 1;
  for (int k = 1; k <= 32 && k * grain <= steps; ++k) {
    if (steps % (k * grain)) continue;
    best = k;
    if (wgs * k >= 1024) break;
  }
  return best;
}

// Reduction parts for the dense path's gate/up GEMM, chosen like the down GEMM's.
int gateup_kparts(const Shape& s, int T) {
  if (!s.dense || use_tiled(s, T)) return 1;
  const int bm = expert_tile_rows(s, T);
  const long wgs = (long)((T + bm - 1) / bm) * ((s.I + 63) / 64);
  const int steps = steps_per_k(s, s.H);
  const int grain = steps % 4 == 0 ? 4 : (steps % 2 == 0 ? 2 : 1);
  int best = 1;
  for (int k = 1; k <= 32 && k * grain <= steps; ++k) {
    if (steps % (k * grain)) continue;
    best = k;
    if (wgs * k >= 1024) break;
  }
  return best;
}

// Dispatch on (weight type, row-tile count, depth).
template <int cap, typename F>
static hipError_t with_depth(int nsteps, F&& f) {
  switch (pick_depth(nsteps, cap)) {
    case 4: return f(std::integral_constant<int, (cap >= 4 ? 4 : 1)>{});
    case 2: return f(std::integral_constant<int, (cap >= 2 ? 2 : 1)>{});
    default: return f(std::integral_constant<int, 1>{});
  }
}

template <typename G>
static hipError_t dispatch_wt_mt(const Shape& s, int bm, G&& go) {
  using M1 = std::integral_constant<int, 1>;
  using M2 = std::integral_constant<int, 2>;
  using M4 = std::integral_constant<int, 4>;
  auto by_mt = [&](auto wt) { return bm == 16 ? go(wt, M1{}) : bm == 32 ? go(wt, M2{}) : go(wt, M4{}); };
  switch (weight_type_of(s)) {
    case kWMX: return by_mt(std::integral_constant<int, kWMX>{});
    case kWFP8: return by_mt(std::integral_constant<int, kWFP8>{});
    default: return by_mt(std::integral_constant<int, kWBF16>{});
  }
}

hipError_t launch_gateup(const Shape& s, int T, const uint16_t* x, const void* wg, const void* wu,
                         const void* sg, const void* su, const int32_t* offsets, const int32_t* sorted_pairs,
                         const int32_t* tiles, const int32_t* ntiles, int max_tiles, int kparts, float* part,
                         uint16_t* h, hipStream_t stream) {
  if (wide_schedule(s, T) != kWideNone)
    return launch_gateup_wide(s, T, x, wg, wu, sg, su, offsets, sorted_pairs, tiles, ntiles, max_tiles, h, stream);
  if (use_tiled(s, T))
    return launch_gateup_tiled(s, x, wg, wu, static_cast<const float*>(sg), static_cast<const float*>(su), offsets,
                               sorted_pairs, tiles, ntiles, max_tiles, expert_tile_rows(s, T), h, stream);
  if (max_tiles > kMaxGridY) return hipErrorInvalidConfiguration;
  const int nrows = T * s.K;
  return dispatch_wt_mt(s, expert_tile_rows(s, T), [&](auto wt, auto mt) {
    constexpr int WT = decltype(wt)::value;
    constexpr int M = decltype(mt)::value;
    hipError_t err = with_depth<StreamShape<WT, M>::kGateUpDepth>(s.H / WFrag<WT>::SK / kparts, [&](auto d) {
      return gateup_launch<WT, M, StreamShape<WT, M>::kGateUpG, decltype(d)::value>(
          s, x, wg, wu, sg, su, offsets, sorted_pairs, tiles, ntiles, max_tiles, h, kparts, nrows, part, stream);
    });
    if (err != hipSuccess || kparts == 1) return err;
    const size_t n4 = (size_t)nrows * s.I / 4;
    const int blocks = (int)std::min<size_t>((n4 + 255) / 256, 4096);
    const float* fsg = WT == kWFP8 ? static_cast<const float*>(sg) : nullptr;   // MXFP4 scales are already applied
    const float* fsu = WT == kWFP8 ? static_cast<const float*>(su) : nullptr;
    hipLaunchKernelGGL(swiglu_reduce_kernel, dim3(blocks), dim3(256), 0, stream, nrows, s.I, kparts, part, fsg, fsu,
                       h);
    return hipGetLastError();
  });
}

hipError_t launch_down(const Shape& s, int T, const uint16_t* h, const void* wd, const void* sd,
                       const int32_t* offsets, const int32_t* tiles, const int32_t* ntiles, int max_tiles,
                       int kparts, float* part, uint16_t* y, hipStream_t stream) {
  if (wide_schedule(s, T) == kWideModerate || (wide_schedule(s, T) == kWideBalanced && s.packed))
    return launch_down_wide(s, T, h, wd, sd, offsets, tiles, ntiles, max_tiles, y, stream);
  if (use_tiled(s, T))
    return launch_down_tiled(s, h, wd, static_cast<const float*>(sd), offsets, tiles, ntiles, max_tiles,
                             expert_tile_rows(s, T), y, stream);
  if (max_tiles > kMaxGridY) return hipErrorInvalidConfiguration;
  const int nrows = T * s.K;
  return dispatch_wt_mt(s, expert_tile_rows(s, T), [&](auto wt, auto mt) {
    constexpr int WT = decltype(wt)::value;
    constexpr int M = decltype(mt)::value;
    hipError_t err = with_depth<StreamShape<WT, M>::kDownDepth>(s.I / WFrag<WT>::SK / kparts, [&](auto d) {
      return down_launch<WT, M, StreamShape<WT, M>::kDownG, decltype(d)::value>(s, h, wd, sd, offsets, tiles, ntiles,
                                                                                 max_tiles, y, kparts, nrows, part,
                                                                                 stream);
    });
    if (err != hipSuccess || kparts == 1) return err;
    const size_t n4 = (size_t)nrows * s.H / 4;
    const int blocks = (int)std::min<size_t>((n4 + 255) / 256, 4096);
    const float* fsd = WT == kWFP8 ? static_cast<const float*>(sd) : nullptr;   // MXFP4 scales are already applied
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, stream, nrows, s.H, kparts, part, fsd, y);
    return hipGetLastError();
  });
}

}  // namespace beam

namespace beam {

// Identity permutation and row tiles of the single expert of the dense path.
__global__ __launch_bounds__(256) void dense_setup_kernel(int T, int tile_rows, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int nt = (T + tile_rows - 1) / tile_rows;
  if (i < T) sorted_pairs[i] = i;
  if (i < nt) {
    tiles[2 * i] = 0;
    tiles[2 * i + 1] = i * tile_rows;
  }
  if (i == 0) {
    offsets[0] = 0;
    offsets[1] = T;
    ntiles[0] = nt;
  }
}

hipError_t launch_dense_setup(int T, int tile_rows, int32_t* offsets, int32_t* sorted_pairs, int32_t* tiles,
                              int32_t* ntiles, hipStream_t stream) {
  hipLaunchKernelGGL(dense_setup_kernel, dim3((T + 255) / 256), dim3(256), 0, stream, T, tile_rows, offsets,
                     sorted_pairs, tiles, ntiles);
  return hipGetLastError();
}

}  // namespace beam
