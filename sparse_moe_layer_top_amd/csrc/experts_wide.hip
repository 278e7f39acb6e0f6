// Gate/up grouped GEMM + SwiGLU for the prefill regime, bf16 weights: one
// workgroup per CU, weights streamed straight into registers.
//
// Same arithmetic as the other expert kernels (each expert a SwiGLU MLP,
// Reflection Beam 1.0 overview, section "Mixture of Experts"; the SwiGLU
// product in FP32, section "Residual stream"):
//   h = bf16( SiLU(x Wg^T) * (x Wu^T) )
//
// At a few hundred rows per expert the GEMM reads each weight byte once and
// does about 250 FLOP per byte: close to the MFMA/HBM balance point, so the
// schedule has to keep HBM streaming while the matrix cores run.  Here:
//
//   * 8 waves (two per SIMD); every wave spans the tile's 272 rows (17 MFMA
//     blocks of 16, a whole balanced expert) and owns 16 intermediate
//     columns: one gate and one up block of 16, 136 accumulator registers.
//     No other wave needs its weight rows.
//   * Each wave's weight rows go HBM -> VGPRs with 16-byte buffer loads into
//     a ring of four 64-k windows, three ahead of the MFMAs (96 KB of
//     weights in flight per CU).
//   * The token rows, needed by every wave, go HBM/L2 -> LDS with
//     direct-to-LDS buffer loads into a ring of four stages, also three
//     windows ahead.  One load instruction covers 8 rows x one row's whole
//     128-byte window slice, lane l taking row l/8 and 16-byte chunk
//     (l%8) ^ (l/8) ^ (group%2), so every MFMA operand reads back with one
//     conflict-free ds_read_b128 (the same swizzle as the LDS-tiled kernels).
//     Groups 0..31 of a window go 4 to each wave, groups 32 and 33 (rows
//     256..271) to waves 0 and 1; groups wholly past the tile's rows are not
//     fetched (their loads read past the buffer's end, which returns zeros
//     without a memory access; the other waves' fifth loads land in two spare
//     slots of the stage).
//   * Lane (r = l%16, q = l/16) of MFMA half a of a window uses k in
//     [16q + 8a, +8) of the window for both operands.
//   * Every row block runs every window (rows past the tile's end hold its
//     last row, zeros or stale values, and are never stored: an MFMA output
//     row depends on its own A row only), so the compute has no branches and
//     reads its activation fragments three blocks ahead of their MFMAs.
//   * Each stage is its own LDS array, so the compiler tells a wave's loads
//     into one stage from reads of another and waits for the former only:
//     before the window's barrier every wave reads back a word of each slot
//     it filled in that stage (the compiler waits for those loads), and the
//     barrier then publishes the stage to every wave; it also says every wave
//     is done with the stage (and the registers) the next issue reuses.
//   * The h tile is staged through LDS and stored as whole 16-byte chunks
//     along rows.
//   * Work items (row tile, column block) are dealt to the 8 XCDs in
//     contiguous ranges, so the workgroups of one expert share its token rows
//     in one L2.
//
// The MFMAs of a window read 17 activation fragments per 34 MFMAs from LDS
// (each fragment feeds a gate and an up block), which bounds the compute
// phase at about 70% of the MFMA rate; the loads overlap it only in part.
#include "common.h"

namespace beam {

constexpr int kWRows = 272;                  // rows per tile
constexpr int kWMBlk = kWRows / 16;          // 17 row blocks
constexpr int kWCols = 128;                  // intermediate columns per tile
constexpr int kWWin = 64;                    // k per window: one 128-byte line of a bf16 row
constexpr int kWAhead = 3;                   // windows in flight ahead of the one multiplied
constexpr int kWRing = kWAhead + 1;          // LDS stages = weight register buffers
constexpr int kWWaves = 8;
constexpr int kWGroups = kWRows / 8;         // 34 activation load groups per window
constexpr int kWGPW = (kWGroups + kWWaves - 1) / kWWaves;   // 5 per wave
constexpr int kWStage = 36 * 1024;           // 34 KB of activations + 2 spare slots; 68 staged output rows
constexpr int kWOutRows = kWRows / kWRing;   // h rows staged per stage array
constexpr int kWXcds = 8;

typedef __attribute__((address_space(3))) void wlds_void;

constexpr int kRsrcWord3 = 0x00020000;       // raw buffer resource, 32-bit data format
constexpr uint32_t kPastEnd = 0x80000000u;   // a buffer offset past every resource's extent (< 2^31)

// Stage accesses name the stage arrays themselves: the compiler gives each LDS variable its own
// alias scope, which lets it match a read of a stage to the direct-to-LDS loads into that stage (and
// not to loads into the others) when it places its waits.
__device__ __forceinline__ void stage_fill(uint8_t* st, __amdgpu_buffer_rsrc_t rsrc, const int (&slot)[kWGPW],
                                           const uint32_t (&off)[kWGPW], int soff) {
#pragma unroll
  for (int i = 0; i < kWGPW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (wlds_void*)(st + slot[i]), 16, off[i], soff, 0, 0);
}
// One word of each of this wave's slots in a stage: the compiler waits for all of the wave's loads into it.
__device__ __forceinline__ uint32_t stage_probe(const uint8_t* st, const int (&slot)[kWGPW], int lane) {
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < kWGPW; ++i) v |= *reinterpret_cast<const uint32_t*>(st + slot[i] + lane * 16);
  return v;
}

// (The weight pointers are not restrict: with them the compiler moves each window's weight loads
// down to their first use, three windows later, which empties the pipeline.)
__global__ __launch_bounds__(512) void wide_gateup_kernel(int H, int I, int K, const uint16_t* __restrict__ x,
                                                          const uint16_t* wg, const uint16_t* wu,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted_pairs,
                                                          const int32_t* __restrict__ tiles,
                                                          const int32_t* __restrict__ ntiles,
                                                          uint16_t* __restrict__ h, long x_bytes) {
  constexpr int CST = kWCols * 2 + 16;                      // staged h row stride, bytes
  static_assert(kWGroups * 1024 + 2048 <= kWStage && kWOutRows * CST <= kWStage, "stage size");
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kWStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kWStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[kWStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[kWStage];
  auto stage = [&](auto sc) -> uint8_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return lds0;
    else if constexpr (S == 1) return lds1;
    else if constexpr (S == 2) return lds2;
    else return lds3;
  };

  const int NT = I / kWCols;                                // column blocks per tile
  const int nitems = ntiles[0] * NT;
  const int per_xcd = (nitems + kWXcds - 1) / kWXcds;
  const int slot = blockIdx.x / kWXcds;
  if (slot >= per_xcd) return;
  const int item = (blockIdx.x % kWXcds) * per_xcd + slot;
  if (item >= nitems) return;
  const int tile = item / NT, jn = item % NT;
  const int e = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int lo = offsets[e];
  const int rows = min(offsets[e + 1] - lo - r0, kWRows);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int l16 = lane % 16, q = lane / 16;

  // Token-row load groups of this wave: g = wave + 8i, rows 8g + lane/8 (clamped to the tile), as
  // byte offsets into a buffer resource over x (below 2^31 bytes, checked by the launcher).  The
  // fifth load: group 32 + wave for waves 0 and 1 of a tile taller than 256 rows; otherwise it reads
  // past the buffer's end (zeros, no memory access) into one of the stage's two spare slots.
  const __amdgpu_buffer_rsrc_t xrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0, (int)x_bytes, kRsrcWord3);
  uint32_t aoff[kWGPW];
  int aslot[kWGPW];
#pragma unroll
  for (int i = 0; i < kWGPW; ++i) {
    const int gw = wave + kWWaves * i;
    const bool live = gw < kWGroups && 8 * gw < rows;
    const int g = gw < kWGroups ? gw : kWGroups + gw % 2;
    aslot[i] = g * 1024;
    const int r = min(8 * g + lane / 8, rows - 1);
    const uint32_t tok = (uint32_t)(sorted_pairs[lo + r0 + r] / K);
    aoff[i] = live ? (tok * (uint32_t)H + ((lane % 8) ^ (lane / 8) ^ (g % 2)) * 8) * 2 : kPastEnd;
  }
  // This wave's gate and up rows (the same intermediate columns), through buffer resources over the
  // expert's two matrices.
  const size_t wmat = (size_t)I * H;   // elements per expert matrix
  const __amdgpu_buffer_rsrc_t grsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wg + e * wmat), (short)0, (int)(wmat * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ursrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wu + e * wmat), (short)0, (int)(wmat * 2), kRsrcWord3);
  const uint32_t woff = ((uint32_t)(jn * kWCols + wave * 16 + l16) * H + 16 * q) * 2;
  // where lane (r, q) finds chunk 2q + a of row r of a 16-row block (two 1 KB groups)
  int roff[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) roff[a] = (l16 / 8) * 1024 + ((l16 % 8) * 8 + ((2 * q + a) ^ (l16 % 8) ^ (l16 / 8))) * 16;

  u32x4 wb[kWRing][2][2];   // [slot][half][gate, up]
  f32x4 acc[kWMBlk][2];
#pragma unroll
  for (int m = 0; m < kWMBlk; ++m) acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nwin = H / kWWin;   // a multiple of kWRing (checked by the launcher)
  // Window win into ring slot S.  Past the end the last window is issued again (into a slot nothing
  // reads): every round issues the same loads.
  auto issue = [&](auto sc, int win) {
    constexpr int S = decltype(sc)::value;
    stage_fill(stage(sc), xrsrc, aslot, aoff, win * kWWin * 2);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      wb[S][a][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(grsrc, woff, win * kWWin * 2 + 16 * a, 0));
      wb[S][a][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ursrc, woff, win * kWWin * 2 + 16 * a, 0));
    }
  };
  auto compute = [&](auto sc) {
    constexpr int S = decltype(sc)::value;
    const uint8_t* st = stage(sc);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int m = 0; m < kWMBlk; ++m) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(st + m * 2048 + roff[a]);
#pragma unroll
        for (int n = 0; n < 2; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, wb[S][a][n]), acc[m][n],
                                                              0, 0, 0);
      }
    }
    constexpr int kAhead = 3;
    constexpr int kReads = 2 * kWMBlk;
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);   // DS reads
#pragma unroll
    for (int i = 0; i < kReads - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);      // MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kAhead, 0);
  };
  // Open window w (ring slot S): this wave's loads into stage S have landed (reading back a word of
  // each slot makes the compiler wait for them), then the barrier: every wave's have, and every wave
  // is done with window w-1, whose stage and registers the next issue reuses.
  auto open = [&](auto sc, int w) {
    constexpr int S = decltype(sc)::value;
    const uint32_t probe = stage_probe(stage(sc), aslot, lane);
    asm volatile("" ::"v"(probe) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(std::integral_constant<int, (S + kWAhead) % kWRing>{}, min(w + kWAhead, nwin - 1));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto run = [&](auto sc) {
    compute(sc);
    __builtin_amdgcn_sched_barrier(0);
  };

  issue(std::integral_constant<int, 0>{}, 0);
  issue(std::integral_constant<int, 1>{}, 1);
  issue(std::integral_constant<int, 2>{}, 2);
  __builtin_amdgcn_sched_barrier(0);
  open(std::integral_constant<int, 0>{}, 0);
  for (int w = 0;; w += kWRing) {   // each round enters after window w's opening
    run(std::integral_constant<int, 0>{});
    open(std::integral_constant<int, 1>{}, w + 1);
    run(std::integral_constant<int, 1>{});
    open(std::integral_constant<int, 2>{}, w + 2);
    run(std::integral_constant<int, 2>{});
    open(std::integral_constant<int, 3>{}, w + 3);
    run(std::integral_constant<int, 3>{});
    if (w + kWRing >= nwin) break;
    open(std::integral_constant<int, 0>{}, w + kWRing);
  }

  // Epilogue: C[r][c] sits in lane (c = l%16, r = 4q + i) of each 16x16 block.  Stage the bf16 h tile
  // row-major in LDS, rows [68j, 68j + 68) in stage j (after the repeated tail loads into stages 0..2
  // have landed and every wave is past the last window), then store whole rows.
  {
    uint32_t probe = 0;
    probe |= stage_probe(lds0, aslot, lane);
    probe |= stage_probe(lds1, aslot, lane);
    probe |= stage_probe(lds2, aslot, lane);
    asm volatile("" ::"v"(probe) : "memory");
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  auto orow = [&](int r) -> uint8_t* {
    const int j = r / kWOutRows, rr = r % kWOutRows;
    uint8_t* b = j == 0 ? lds0 : j == 1 ? lds1 : j == 2 ? lds2 : lds3;
    return b + rr * CST;
  };
  const int nmb = (rows + 15) / 16;
  const int c = wave * 16 + l16;
#pragma unroll
  for (int m = 0; m < kWMBlk; ++m) {
    if (m < nmb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m * 16 + q * 4 + i;
        *reinterpret_cast<uint16_t*>(orow(r) + c * 2) = f32_to_bf16(silu(acc[m][0][i]) * acc[m][1][i]);
      }
    }
  }
  __syncthreads();
  constexpr int CPR = kWCols / 8;   // 16-byte chunks per h row
  uint16_t* const obase = h + (size_t)(lo + r0) * I + (size_t)jn * kWCols;
  for (int idx = threadIdx.x; idx < rows * CPR; idx += kWWaves * kWave) {
    const int r = idx / CPR, ch = idx % CPR;
    *reinterpret_cast<u32x4*>(obase + (size_t)r * I + ch * 8) = *reinterpret_cast<const u32x4*>(orow(r) + ch * 16);
  }
}

// bf16 MoE layers in the tiled regime with balanced loads (at least 3/4 of a 256-row expert per
// expert on average; with fewer rows the LDS-tiled kernel, which skips empty row blocks, does as
// well), whose reduction is whole rounds of the window ring and whose token rows fit one buffer
// resource (byte offsets below 2^31).
bool use_wide(const Shape& s, int T) {
  if (s.fp8 || s.mx || s.dense) return false;
  if (!use_tiled(s, T)) return false;
  if ((long)T * s.K < 192L * s.E) return false;
  if ((long)T * s.H * 2 >= (1L << 31)) return false;
  return s.H % (kWWin * kWRing) == 0 && s.I % kWCols == 0;
}

int wide_tile_rows() { return kWRows; }

hipError_t launch_gateup_wide(const Shape& s, int T, const uint16_t* x, const void* wg, const void* wu,
                              const int32_t* offsets, const int32_t* sorted_pairs, const int32_t* tiles,
                              const int32_t* ntiles, int max_tiles, uint16_t* h, hipStream_t stream) {
  if (!use_wide(s, T)) return hipErrorInvalidValue;
  const long items = (long)max_tiles * (s.I / kWCols);
  const int grid = (int)((items + kWXcds - 1) / kWXcds * kWXcds);
  hipLaunchKernelGGL(wide_gateup_kernel, dim3(grid), dim3(kWWaves * kWave), 0, stream, s.H, s.I, s.K, x,
                     static_cast<const uint16_t*>(wg), static_cast<const uint16_t*>(wu), offsets, sorted_pairs, tiles,
                     ntiles, h, (long)T * s.H * 2);
  return hipGetLastError();
}

}  // namespace beam
