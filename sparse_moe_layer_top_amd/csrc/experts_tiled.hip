// Grouped SwiGLU expert GEMMs for large token counts: LDS-tiled bf16 MFMA.
//
// Same arithmetic as the weight-streaming kernels (each expert a SwiGLU MLP,
// Reflection Beam 1.0 overview, section "Mixture of Experts"; the SwiGLU
// product in FP32, section "Residual stream"), scheduled for the prefill
// regime where an expert holds hundreds of rows:
//
//   * A workgroup owns one row tile of an expert (up to 288 rows, 18 blocks of
//     16) and 256 weight rows (gate/up: 128 gate + the matching 128 up rows,
//     so the SwiGLU epilogue stays in registers; down: 256 output columns).
//     With 288 rows a whole expert of the balanced prefill fits one tile, so
//     every weight byte comes from HBM once.
//   * Operands move HBM/L2 -> LDS with direct-to-LDS 16-byte loads
//     (global_load_lds_dwordx4).  One load instruction covers 8 rows x the
//     row's whole 128-byte stage slice (8 full cache lines): lane l takes row
//     l/8 and 16-byte chunk (l%8) ^ (l/8) ^ j, j the instruction's half of a
//     16-row block.  That XOR swizzle lets each lane read its MFMA operand back
//     with one conflict-free ds_read_b128: lane (r = l%16, q = l/16) of half
//     a = 0, 1 needs k in [16q + 8a, +8) of the 64-wide stage, i.e. chunk
//     2q + a of row r.  (Loading 16 rows x 64 bytes per instruction, the
//     natural fragment order, touches twice the cache lines and halves the
//     rate at which a CU's loads complete.)  FP8 weights keep 16 e4m3 bytes
//     per lane (both halves, 16 rows x 64 bytes) and are converted to bf16
//     when read from LDS; the k mapping is the same.  Weights in fragment
//     order (1 KB lane-ordered 64-byte column slices of 16-row blocks) arrive
//     as whole slices, 1 KB of consecutive addresses per instruction, and land
//     in LDS in that order: a bf16 lane reads chunk 2(q%2) + a of slice q/2.
//   * Two LDS stages: stage s+1 streams in while stage s feeds the MFMAs.
//   * 8 waves as 2 (rows) x 4 (columns); a wave owns 9 row blocks x 4 column
//     blocks of 16x16x32 MFMA accumulators.  Row blocks past the tile's rows
//     are neither loaded nor multiplied.
//   * The output tile is staged through LDS and written with 16-byte stores
//     along rows (whole 128-byte lines), not the MFMA layout's 32-byte pieces.
//   * Work items (tile, column block) are dealt to the 8 XCDs in contiguous
//     ranges, so the workgroups running together on one XCD share the same
//     expert's activation rows in that XCD's L2.
#include "common.h"

namespace beam {

constexpr int kTM = 288;            // rows per tile
constexpr int kTN = 256;            // weight rows per tile
constexpr int kBK = 64;             // k per LDS stage
constexpr int kMBlk = kTM / 16;     // 18 row blocks
constexpr int kNBlk = kTN / 16;     // 16 weight-row blocks
constexpr int kXcds = 8;

enum { kGateUp = 0, kDown = 1 };

// NBW: weight-row blocks of 16 per column wave (4 waves): 4 (256 weight rows per tile) or, for the
// bf16 down GEMM, 5 (320 output columns: each 64-k stage then brings 36 KB of h rows per 40 KB of
// weights instead of per 32 KB, and its MFMAs take a quarter longer to cover the next stage's loads).
template <bool FP8, int NBW = 4>
struct TiledGeom {
  static constexpr int NBLK = 4 * NBW;                   // weight-row blocks per tile
  static constexpr int TN = 16 * NBLK;                   // weight rows per tile
  static constexpr int A_FR = kMBlk * 2;                 // A fragments per stage
  static constexpr int B_FR = NBLK * (FP8 ? 1 : 2);      // B fragments per stage
  static constexpr int FR = A_FR + B_FR;
  static constexpr int STAGE = FR * 1024;                // bytes per stage
  static constexpr int LPW = (FR + 7) / 8;               // fragment loads per wave per stage
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void load_lds16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_base, 16, 0, 0);
}

template <int MODE, bool FP8, int NBW>
__global__ __launch_bounds__(512) void tiled_kernel(int H, int I, int K, const uint16_t* __restrict__ act,
                                                    const void* __restrict__ w0, const void* __restrict__ w1,
                                                    const float* __restrict__ s0, const float* __restrict__ s1,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ sorted_pairs,
                                                    const int32_t* __restrict__ tiles,
                                                    const int32_t* __restrict__ ntiles, uint16_t* __restrict__ out,
                                                    int tile_rows, int packed) {
  using G = TiledGeom<FP8, NBW>;
  static_assert(MODE == kDown || NBW == 4, "gate/up pairs 2 gate + 2 up blocks per wave");
  constexpr int NC = MODE == kGateUp ? 128 : G::TN;      // output columns per tile
  constexpr int CST = NC * 2 + 16;                        // staged output row stride in bytes
  // the output tile goes out in EP passes of kTM / EP rows when it does not fit the two stages
  constexpr int EP = kTM * CST <= 2 * G::STAGE ? 1 : 2;
  constexpr int LDS = (2 * G::STAGE > kTM / EP * CST) ? 2 * G::STAGE : kTM / EP * CST;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];

  const int NT = MODE == kGateUp ? I / 128 : H / G::TN;   // column blocks per tile
  const int KD = MODE == kGateUp ? H : I;                 // reduction length
  const int nitems = ntiles[0] * NT;
  const int per_xcd = (nitems + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int item = (blockIdx.x % kXcds) * per_xcd + slot;
  if (item >= nitems) return;
  const int tile = item / NT, jn = item % NT;
  const int e = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int lo = offsets[e];
  const int rows = min(offsets[e + 1] - lo - r0, tile_rows);   // tile_rows <= kTM (checked by the launchers)
  const int nmb = (rows + 15) / 16;

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int l16 = lane % 16, q = lane / 16;
  const int wm = wave / 4, wn = wave % 4;
  constexpr int WB = FP8 ? 1 : 2;                          // bytes per weight element
  const int lrow = lane / 8, lchunk = (lane % 8) ^ (lane / 8);

  // the load instructions this wave issues every stage: f = wave + 8*i
  const uint8_t* src[G::LPW];
  bool on[G::LPW];
#pragma unroll
  for (int i = 0; i < G::LPW; ++i) {
    const int f = wave + 8 * i;
    on[i] = f < G::FR;
    src[i] = nullptr;
    if (!on[i]) continue;
    if (f < G::A_FR) {
      const int mb = f / 2, j = f % 2;
      on[i] = mb < nmb;
      const int r = min(mb * 16 + j * 8 + lrow, rows - 1);
      const size_t row = MODE == kGateUp ? (size_t)(sorted_pairs[lo + r0 + r] / K) : (size_t)(lo + r0 + r);
      src[i] = reinterpret_cast<const uint8_t*>(act + row * KD + (lchunk ^ j) * 8);
    } else {
      const int fb = f - G::A_FR;
      const int nb = FP8 ? fb : fb / 2, j = FP8 ? 0 : fb % 2;
      const void* wbase;
      size_t wrow0;                                        // the 16-row weight block's first row
      if (MODE == kGateUp) {
        wbase = nb < 8 ? w0 : w1;
        wrow0 = (size_t)e * I + jn * 128 + (nb % 8) * 16;
      } else {
        wbase = w0;
        wrow0 = (size_t)e * H + jn * G::TN + nb * 16;
      }
      if (packed) {   // slice j of the block's stage (bf16: two 64-byte slices per 128-byte stage)
        src[i] = static_cast<const uint8_t*>(wbase) + wrow0 * KD * WB + j * 1024 + lane * 16;
      } else {
        const int rib = FP8 ? l16 : j * 8 + lrow;            // row inside the 16-row weight block
        const size_t k0 = FP8 ? (size_t)q * 16 : (size_t)(lchunk ^ j) * 8;
        src[i] = static_cast<const uint8_t*>(wbase) + ((wrow0 + rib) * KD + k0) * WB;
      }
    }
  }
  // bytes between stages: activation rows and row-order weights advance along the row; fragment-order
  // weights by the 16 rows' stage slices
  const size_t wstep = packed ? (size_t)16 * kBK * WB : (size_t)kBK * WB;
  auto issue = [&](int stage, int buf) {
#pragma unroll
    for (int i = 0; i < G::LPW; ++i) {
      if (!on[i]) continue;   // wave-uniform
      const int f = wave + 8 * i;
      const size_t step = (size_t)stage * (f < G::A_FR ? kBK * 2 : wstep);
      load_lds16(src[i] + step, smem + buf * G::STAGE + f * 1024);
    }
  };

  // where lane (r, q) finds chunk 2q + a of row r of a 16-row block (two 1 KB load instructions), and
  // its bf16 weight operand of half a (row order: the same; fragment order: chunk 2(q%2) + a of slice q/2)
  int roff[2], wro[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    roff[a] = (l16 / 8) * 1024 + ((l16 % 8) * 8 + ((2 * q + a) ^ (l16 % 8) ^ (l16 / 8))) * 16;
    wro[a] = packed ? (q / 2) * 1024 + (l16 + 16 * (2 * (q % 2) + a)) * 16 : roff[a];
  }

  // this wave's weight-row blocks: gate/up pairs for the SwiGLU, or NBW down blocks
  int nbs[NBW];
#pragma unroll
  for (int n = 0; n < NBW; ++n)
    nbs[n] = MODE == kGateUp ? ((n < 2) ? 2 * wn + n : 8 + 2 * wn + (n - 2)) : NBW * wn + n;

  f32x4 acc[9][NBW];
#pragma unroll
  for (int m = 0; m < 9; ++m)
#pragma unroll
    for (int n = 0; n < NBW; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int kWaitLoads = (7 << 4) | (15 << 8);        // s_waitcnt vmcnt(0)
  const int nst = KD / kBK;
  issue(0, 0);
  for (int s = 0; s < nst; ++s) {
    const int buf = s & 1;
    __builtin_amdgcn_s_waitcnt(kWaitLoads);             // this wave's loads of stage s have landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();                       // ... and every other wave's; stage s-1 fully read
    asm volatile("" ::: "memory");
    if (s + 1 < nst) issue(s + 1, buf ^ 1);
    const uint8_t* st = smem + buf * G::STAGE;
    u32x4 braw[NBW];
    if constexpr (FP8) {
#pragma unroll
      for (int n = 0; n < NBW; ++n)
        braw[n] = *reinterpret_cast<const u32x4*>(st + (G::A_FR + nbs[n]) * 1024 + lane * 16);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      bf16x8 b[NBW];
#pragma unroll
      for (int n = 0; n < NBW; ++n) {
        if constexpr (FP8) {
          b[n] = e4m3x8_to_bf16x8(a == 0 ? u32x2{braw[n][0], braw[n][1]} : u32x2{braw[n][2], braw[n][3]});
        } else {
          b[n] = *reinterpret_cast<const bf16x8*>(st + (G::A_FR + nbs[n] * 2) * 1024 + wro[a]);
        }
      }
#pragma unroll
      for (int m = 0; m < 9; ++m) {
        const int mb = wm * 9 + m;
        if (mb < nmb) {   // wave-uniform
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(st + mb * 2048 + roff[a]);
#pragma unroll
          for (int n = 0; n < NBW; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[n], acc[m][n], 0, 0, 0);
        }
      }
    }
  }

  // epilogue: C[r][c] sits in lane (c = l%16, r = 4q + i) of each 16x16 block; stage the bf16 tile
  // row-major in LDS (every wave is done with the last stage first), then store whole rows; with
  // EP = 2, the row half of waves wm = p goes out in pass p
  constexpr int CPR = NC / 8;                               // 16-byte chunks per output row
  const int ldo = MODE == kGateUp ? I : H;
  uint16_t* const obase = out + (size_t)(lo + r0) * ldo + (size_t)jn * NC;
#pragma unroll
  for (int p = 0; p < EP; ++p) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int rbase = p * (kTM / EP);                      // first row staged in this pass
    if (EP == 1 || wm == p) {
      if constexpr (MODE == kGateUp) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int c = (2 * wn + n) * 16 + l16;
          const float sg = FP8 ? s0[(size_t)e * I + jn * 128 + c] : 1.f;
          const float su = FP8 ? s1[(size_t)e * I + jn * 128 + c] : 1.f;
#pragma unroll
          for (int m = 0; m < 9; ++m) {
            if (wm * 9 + m < nmb) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int r = (wm * 9 + m) * 16 + q * 4 + i;
                const float g = acc[m][n][i] * sg, u = acc[m][n + 2][i] * su;
                *reinterpret_cast<uint16_t*>(smem + (r - rbase) * CST + c * 2) = f32_to_bf16(silu(g) * u);
              }
            }
          }
        }
      } else {
#pragma unroll
        for (int n = 0; n < NBW; ++n) {
          const int c = (NBW * wn + n) * 16 + l16;
          const float sd = FP8 ? s0[(size_t)e * H + jn * G::TN + c] : 1.f;
#pragma unroll
          for (int m = 0; m < 9; ++m) {
            if (wm * 9 + m < nmb) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int r = (wm * 9 + m) * 16 + q * 4 + i;
                *reinterpret_cast<uint16_t*>(smem + (r - rbase) * CST + c * 2) = f32_to_bf16(acc[m][n][i] * sd);
              }
            }
          }
        }
      }
    }
    __syncthreads();
    const int prow = min(rows - rbase, kTM / EP);           // rows of this pass that exist
    for (int idx = threadIdx.x; idx < prow * CPR; idx += 512) {
      const int r = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<u32x4*>(obase + (size_t)(rbase + r) * ldo + ch * 8) =
          *reinterpret_cast<const u32x4*>(smem + r * CST + ch * 16);
    }
  }
}

bool use_tiled(const Shape& s, int T) {
  // a single expert gives the tiled kernels only ceil(T/288) row tiles: below ~1k
  // tokens the streaming kernels (64-row tiles, k-split down) fill the chip better
  if (s.dense && T <= 1024) return false;
  if (s.mx) return false;   // MXFP4 never takes these kernels (one-workgroup-per-CU or streaming kernels)
  const long mean = ((long)T * s.K) / s.E;
  return mean >= 32 && s.H % kTN == 0 && s.I % 128 == 0;
}

int tiled_tile_rows() { return kTM; }

static int grid_for(int max_tiles, int nt) {
  const long items = (long)max_tiles * nt;
  return (int)((items + kXcds - 1) / kXcds * kXcds);
}

hipError_t launch_gateup_tiled(const Shape& s, const uint16_t* x, const void* wg, const void* wu, const float* sg,
                               const float* su, const int32_t* offsets, const int32_t* sorted_pairs,
                               const int32_t* tiles, const int32_t* ntiles, int max_tiles, int tile_rows, uint16_t* h,
                               hipStream_t stream) {
  if (tile_rows < 1 || tile_rows > kTM) return hipErrorInvalidValue;
  const dim3 grid(grid_for(max_tiles, s.I / 128));
  if (s.fp8)
    hipLaunchKernelGGL((tiled_kernel<kGateUp, true, 4>), grid, dim3(512), 0, stream, s.H, s.I, s.K, x, wg, wu, sg, su,
                       offsets, sorted_pairs, tiles, ntiles, h, tile_rows, s.packed);
  else
    hipLaunchKernelGGL((tiled_kernel<kGateUp, false, 4>), grid, dim3(512), 0, stream, s.H, s.I, s.K, x, wg, wu, sg, su,
                       offsets, sorted_pairs, tiles, ntiles, h, tile_rows, s.packed);
  return hipGetLastError();
}

hipError_t launch_down_tiled(const Shape& s, const uint16_t* h, const void* wd, const float* sd,
                             const int32_t* offsets, const int32_t* tiles, const int32_t* ntiles, int max_tiles,
                             int tile_rows, uint16_t* y, hipStream_t stream) {
  if (tile_rows < 1 || tile_rows > kTM) return hipErrorInvalidValue;
  if (s.fp8) {
    hipLaunchKernelGGL((tiled_kernel<kDown, true, 4>), dim3(grid_for(max_tiles, s.H / kTN)), dim3(512), 0, stream,
                       s.H, s.I, s.K, h, wd, nullptr, sd, nullptr, offsets, nullptr, tiles, ntiles, y, tile_rows,
                       s.packed);
  } else if (s.H % TiledGeom<false, 5>::TN == 0) {
    hipLaunchKernelGGL((tiled_kernel<kDown, false, 5>), dim3(grid_for(max_tiles, s.H / TiledGeom<false, 5>::TN)),
                       dim3(512), 0, stream, s.H, s.I, s.K, h, wd, nullptr, sd, nullptr, offsets, nullptr, tiles,
                       ntiles, y, tile_rows, s.packed);
  } else {
    hipLaunchKernelGGL((tiled_kernel<kDown, false, 4>), dim3(grid_for(max_tiles, s.H / kTN)), dim3(512), 0, stream,
                       s.H, s.I, s.K, h, wd, nullptr, sd, nullptr, offsets, nullptr, tiles, ntiles, y, tile_rows,
                       s.packed);
  }
  return hipGetLastError();
}

}  // namespace beam
